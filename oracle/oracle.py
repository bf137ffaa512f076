"""ctypes wrapper of the C oracle (fp4_oracle.c).

Test infrastructure only.  Every function takes numpy arrays (or torch CPU
tensors, converted exactly to binary32) and returns numpy arrays.  Nothing here
touches a GPU or the GPU library.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_lib")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")

__all__ = [
    "build", "lib", "e2m1_value", "e4m3_value", "e4m3_encode", "e2m1_encode", "recip",
    "round_fp16", "quantize_block", "quantize", "dequantize", "block_means", "block_scores", "block_topk",
    "topk_count", "attention_fwd", "attention_exact", "attention_decode", "num_threads", "balance_exponents",
    "balance_apply",
    "score_factor", "kv_append", "block_sums", "hadamard_rows", "attention_train", "mx_quantize",
    "mx_dequantize", "mx_scale_byte",
]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no contraction of multiply-adds)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_vp = C.c_void_p


def lib():
    global _lib
    if _lib is not None:
        return _lib
    path = build()
    L = C.CDLL(path)
    L.orc_e2m1_value.argtypes = [C.c_int]; L.orc_e2m1_value.restype = C.c_double
    L.orc_e4m3_value.argtypes = [C.c_int]; L.orc_e4m3_value.restype = C.c_double
    L.orc_e4m3_encode.argtypes = [C.c_double]; L.orc_e4m3_encode.restype = C.c_int
    L.orc_e2m1_encode.argtypes = [C.c_double]; L.orc_e2m1_encode.restype = C.c_int
    L.orc_recip.argtypes = [C.c_int]; L.orc_recip.restype = C.c_float
    L.orc_round_fp16.argtypes = [C.c_double]; L.orc_round_fp16.restype = C.c_double
    L.orc_score_factor.argtypes = [C.c_double, C.c_int]; L.orc_score_factor.restype = C.c_float
    L.orc_quantize_block.argtypes = [_f32p, C.c_int, C.c_int, C.c_int, C.c_int, _u8p,
                                     _u8p, _i8p, _vp]
    L.orc_quantize_block.restype = C.c_int
    L.orc_quantize.argtypes = [_f32p, C.c_int64, C.c_int64, C.c_int, C.c_int, C.c_int, C.c_int,
                               C.c_int, C.POINTER(C.c_float), _u8p, _u8p, _vp]
    L.orc_quantize.restype = C.c_int64
    L.orc_dequantize.argtypes = [_u8p, _u8p, C.c_int64, C.c_int64, C.c_int, C.c_float, _f64p]
    L.orc_dequantize.restype = None
    L.orc_block_means.argtypes = [_f32p, C.c_int64, C.c_int, C.c_int, _f64p]
    L.orc_block_means.restype = None
    L.orc_topk_count.argtypes = [C.c_int, C.c_int]; L.orc_topk_count.restype = C.c_int
    L.orc_block_topk.argtypes = [_f64p, _f64p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                 C.c_int, _i32p, _i32p]
    L.orc_block_topk.restype = None
    L.orc_block_scores.argtypes = [_f64p, _f64p, C.c_int, C.c_int, C.c_int, _f64p]
    L.orc_block_scores.restype = None
    L.orc_attention_fwd.argtypes = [_f32p, _f32p, _f32p, C.c_int, C.c_int, C.c_int, C.c_int64,
                                    C.c_int64, C.c_int, C.c_int, C.c_double, C.c_int, C.c_int,
                                    C.c_int, C.c_int, C.c_int, C.c_int, _vp, C.c_int64, _vp,
                                    C.c_int, _f32p, _vp, _vp, _vp, _vp, _vp, C.c_int, _vp, _vp, C.c_int,
                                    _vp, _vp]
    L.orc_attention_fwd.restype = C.c_int
    L.orc_mx_scale_byte.argtypes = [C.c_double]; L.orc_mx_scale_byte.restype = C.c_int
    L.orc_mx_quantize.argtypes = [_f32p, C.c_int64, C.c_int64, C.c_int, _u8p, _u8p]
    L.orc_mx_quantize.restype = None
    L.orc_mx_dequantize.argtypes = [_u8p, _u8p, C.c_int64, C.c_int64, C.c_int, _f64p]
    L.orc_mx_dequantize.restype = None
    L.orc_hadamard_rows.argtypes = [_f32p, C.c_int64, C.c_int, _vp]
    L.orc_hadamard_rows.restype = None
    L.orc_balance_exponents.argtypes = [_f32p, _f32p, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int,
                                        _i32p]
    L.orc_balance_exponents.restype = None
    L.orc_attention_exact.argtypes = [_f32p, _f32p, _f32p, C.c_int, C.c_int, C.c_int, C.c_int64,
                                      C.c_int64, C.c_int, C.c_int, C.c_double, _vp, C.c_int64,
                                      _vp, C.c_int, _f32p, _vp]
    L.orc_attention_exact.restype = C.c_int
    L.orc_attention_decode.argtypes = [_f32p, _f32p, _f32p, _i32p, C.c_int, C.c_int, C.c_int,
                                       C.c_int, C.c_int64, C.c_int, C.c_int, C.c_double, C.c_int,
                                       C.c_int, C.c_int, _vp, C.c_int, _f32p, _vp, C.c_int,
                                       C.c_int, C.c_int, _vp, _vp]
    L.orc_attention_decode.restype = C.c_int
    L.orc_block_sums.argtypes = [_f32p, C.c_int64, C.c_int, C.c_int, _f64p]
    L.orc_block_sums.restype = None
    L.orc_num_threads.argtypes = []; L.orc_num_threads.restype = C.c_int
    _lib = L
    return L


def _f32(x) -> np.ndarray:
    """Exact binary32 copy of a numpy array or torch CPU tensor (bf16/fp16/fp32)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(int(byte))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e2m1_encode(t: float) -> int:
    return lib().orc_e2m1_encode(float(t))


def recip(byte: int) -> float:
    return lib().orc_recip(int(byte))


def round_fp16(x: float) -> float:
    return lib().orc_round_fp16(float(x))


def score_factor(softmax_scale: float, d: int) -> float:
    return lib().orc_score_factor(float(softmax_scale), int(d))


def num_threads() -> int:
    return lib().orc_num_threads()


def quantize_block(y, scale_search=True, fmin=-2, fmax=6, return_sse=False):
    """Quantize 16 values; returns (codes[16] unpacked, scale byte, offset[, sse per f])."""
    y = _f32(y).reshape(16)
    codes = np.zeros(16, np.uint8)
    sc = np.zeros(1, np.uint8)
    of = np.zeros(1, np.int8)
    sse = np.zeros(fmax - fmin + 1, np.float32)
    lib().orc_quantize_block(y, 1, int(scale_search), fmin, fmax, codes, sc, of, _ptr(sse))
    out = (codes, int(sc[0]), int(of[0]))
    return out + (sse,) if return_sse else out


def hadamard_rows(x, signs=None):
    """Incoherence processing of the rows of x [..., n] (n a power of two):
    H_n (s o row) / sqrt(n) in binary32 (orc_hadamard_rows); signs is a
    sequence of 32-bit words, bit j set negating element j first."""
    x = _f32(x).copy()
    n = x.shape[-1]
    sg = None if signs is None else np.ascontiguousarray(np.asarray(signs, np.uint32).reshape(-1))
    if sg is not None:
        assert sg.size * 32 >= n
    lib().orc_hadamard_rows(x.reshape(-1), x.size // n, n, _ptr(sg))
    return x


def balance_exponents(q, k):
    """Exponents e [B, Hkv, d] (int32) of the diagonal power-of-two pair
    Q' = Q 2^-e, K' = K 2^e (orc_balance_exponents): per (batch, kv head) and
    channel, the integer in [-8, 8] minimizing ms_q 4^-e + ms_k 4^e."""
    q, k = _f32(q), _f32(k)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    e = np.zeros(B * Hkv * d, np.int32)
    lib().orc_balance_exponents(q.reshape(-1), k.reshape(-1), B, H, Hkv, Sq, Sk, d, e)
    return e.reshape(B, Hkv, d)


def balance_apply(q, k, e):
    """Q' = Q 2^-e and K' = K 2^e in binary32 (exact away from overflow and
    underflow); the exponent vector of kv head h serves its query heads."""
    q, k = _f32(q), _f32(k)
    G = q.shape[1] // k.shape[1]
    eq = np.repeat(e, G, axis=1)[:, :, None, :]
    return np.ldexp(q, -eq).astype(np.float32), np.ldexp(k, e[:, :, None, :]).astype(np.float32)


def mx_quantize(x, block_axis=0):
    """MXFP4 quantization (orc_mx_quantize): blocks of 32, E8M0 scale bytes.
    Returns dict(codes, scales) with layouts like quantize()'s (scales per 32)."""
    x = _f32(x)
    assert x.ndim == 2
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2) if block_axis == 0 else (rows // 2, cols), np.uint8)
    scales = np.zeros((rows, cols // 32) if block_axis == 0 else (rows // 32, cols), np.uint8)
    lib().orc_mx_quantize(np.ascontiguousarray(x).reshape(-1), rows, cols, block_axis, codes.reshape(-1),
                          scales.reshape(-1))
    return dict(codes=codes, scales=scales)


def mx_dequantize(codes, scales, rows, cols, block_axis=0):
    out = np.zeros(rows * cols, np.float64)
    lib().orc_mx_dequantize(np.ascontiguousarray(codes, np.uint8).reshape(-1),
                            np.ascontiguousarray(scales, np.uint8).reshape(-1), rows, cols, block_axis, out)
    return out.reshape(rows, cols)


def mx_scale_byte(a: float) -> int:
    return lib().orc_mx_scale_byte(float(a))


def quantize(x, block_axis=0, scale_search=True, fmin=-2, fmax=6, global_mode=0, g=1.0):
    """Quantize a 2-D tensor. Returns dict(codes, scales, offsets, g, nonfinite_blocks)."""
    x = _f32(x)
    assert x.ndim == 2
    rows, cols = x.shape
    codes = np.zeros(rows * cols // 2, np.uint8)
    scales = np.zeros(rows * cols // 16, np.uint8)
    offs = np.zeros(rows * cols // 16, np.int8)
    gg = C.c_float(g)
    nb = lib().orc_quantize(x, rows, cols, block_axis, int(scale_search), fmin, fmax, global_mode,
                            C.byref(gg), codes, scales, _ptr(offs))
    if nb < 0:
        raise ValueError("bad quantize arguments")
    if block_axis == 0:
        codes = codes.reshape(rows, cols // 2)
        scales = scales.reshape(rows, cols // 16)
        offs = offs.reshape(rows, cols // 16)
    else:
        codes = codes.reshape(rows // 2, cols)
        scales = scales.reshape(rows // 16, cols)
        offs = offs.reshape(rows // 16, cols)
    return dict(codes=codes, scales=scales, offsets=offs, g=gg.value, nonfinite_blocks=int(nb))


def dequantize(codes, scales, rows, cols, block_axis=0, g=1.0):
    out = np.zeros(rows * cols, np.float64)
    lib().orc_dequantize(np.ascontiguousarray(codes, np.uint8).reshape(-1),
                         np.ascontiguousarray(scales, np.uint8).reshape(-1), rows, cols,
                         block_axis, g, out)
    return out.reshape(rows, cols)


def block_means(x, blk=128):
    x = _f32(x)
    S, d = x.shape
    nb = (S + blk - 1) // blk
    out = np.zeros(nb * d, np.float64)
    lib().orc_block_means(x, S, d, blk, out)
    return out.reshape(nb, d)


def topk_count(pct: int, n: int) -> int:
    return lib().orc_topk_count(int(pct), int(n))


def block_scores(qm, km):
    """Scores of every (query block, key block) pair [nqb, nkb] (ThriftAttention
    page, Metodologia / 1): binary64 dot products of the block means, one fused
    multiply-add per channel in ascending order."""
    qm = np.ascontiguousarray(qm, np.float64)
    km = np.ascontiguousarray(km, np.float64)
    out = np.zeros((qm.shape[0], km.shape[0]), np.float64)
    lib().orc_block_scores(qm.reshape(-1), km.reshape(-1), qm.shape[0], km.shape[0], qm.shape[1], out.reshape(-1))
    return out


def block_topk(qm, km, causal, pct):
    qm = np.ascontiguousarray(qm, np.float64)
    km = np.ascontiguousarray(km, np.float64)
    nqb, d = qm.shape
    nkb = km.shape[0]
    kmax = topk_count(pct, nkb)
    idx = np.zeros(max(nqb * kmax, 1), np.int32)
    cnt = np.zeros(nqb, np.int32)
    lib().orc_block_topk(qm.reshape(-1), km.reshape(-1), nqb, nkb, d, int(causal), int(pct), kmax,
                         idx, cnt)
    return idx[: nqb * kmax].reshape(nqb, kmax), cnt


def _sel(arr, dtype):
    if arr is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(arr, dtype=dtype).reshape(-1))
    return a, a.size


def attention_fwd(q, k, v, causal=False, softmax_scale=0.0, kv_tile=128, scale_search=True,
                  fmin=-2, fmax=6, pct=0, sel_block=128, rows=None, heads=None,
                  with_topk=False, hadamard=False, signs=None, single_level_p=False, with_probs=False,
                  mx=False, tie_slack=None, balance=False):
    """Fake-quant FP4 attention. q [B,H,Sq,d], k/v [B,Hkv,Sk,d].

    hadamard: the FP4 path quantizes Q and K after incoherence processing
    (hadamard_rows with the given signs); the FP16 path and the block means
    use the original Q and K.  balance: the FP4 path quantizes Q 2^-e and
    K 2^e (balance_exponents, balance_apply), before the rotation when both
    are on; the FP16 path and the block means again use the originals.  single_level_p quantizes P with the block
    scale alone, E4M3(amax(e)/6) per 16 keys, without the row level.
    mx: the MXFP4 variant (mx_quantize for Q, K, V; P in 32-key blocks with
    the same power-of-two scale rule).  with_probs also returns every row's
    normalized probabilities P and the
    normalized weights P^ the output uses (float64 [nh, nr, Sk] each), after
    the other results.

    tie_slack = (a, b): also return, last, every row's rounding-ambiguity
    bound amb [nh, nr] (float64): how far the row's output (max-abs over d)
    can move when a P code or block scale whose binary32 input lies within the
    relative slack a + b (|tm| + |lg| + |z|) of a rounding boundary is decided
    the other way (see attn_row in fp4_oracle.c).

    Returns (out [nh, nr, d], lse [nh, nr]) and, with with_topk, also
    (topk_idx [nh, nqb, kmax], topk_cnt [nh, nqb])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    qr = kr = None
    qb, kb = q, k
    if balance:
        qb, kb = balance_apply(q, k, balance_exponents(q, k))
        qr, kr = np.ascontiguousarray(qb.reshape(-1)), np.ascontiguousarray(kb.reshape(-1))
    if hadamard:
        qr = np.ascontiguousarray(hadamard_rows(qb, signs).reshape(-1))
        kr = np.ascontiguousarray(hadamard_rows(kb, signs).reshape(-1))
    ra, nr = _sel(rows, np.int64)
    ha, nh = _sel(heads, np.int32)
    nr = nr if ra is not None else Sq
    nh = nh if ha is not None else B * H
    out = np.zeros(nh * nr * d, np.float32)
    lse = np.zeros(nh * nr, np.float32)
    nqb = (Sq + sel_block - 1) // sel_block
    nkb = (Sk + sel_block - 1) // sel_block
    kmax = topk_count(pct, nkb) if pct > 0 else 0
    probs = np.zeros(nh * nr * Sk, np.float64) if with_probs else None
    probs_hat = np.zeros(nh * nr * Sk, np.float64) if with_probs else None
    tidx = np.zeros(max(nh * nqb * kmax, 1), np.int32) if with_topk and pct > 0 else None
    tcnt = np.zeros(max(nh * nqb, 1), np.int32) if with_topk and pct > 0 else None
    tie = np.ascontiguousarray(np.asarray(tie_slack, np.float64)) if tie_slack is not None else None
    amb = np.zeros(nh * nr, np.float64) if tie_slack is not None else None
    rc = lib().orc_attention_fwd(q.reshape(-1), k.reshape(-1), v.reshape(-1), B, H, Hkv, Sq, Sk, d,
                                 int(causal), float(softmax_scale), kv_tile, int(scale_search),
                                 fmin, fmax, int(pct), sel_block, _ptr(ra), nr if ra is not None else 0,
                                 _ptr(ha), nh if ha is not None else 0, out, _ptr(lse), _ptr(tidx),
                                 _ptr(tcnt), _ptr(qr), _ptr(kr), int(bool(single_level_p)),
                                 _ptr(probs), _ptr(probs_hat), int(bool(mx)), _ptr(tie), _ptr(amb))
    if rc != 0:
        raise ValueError("bad attention arguments")
    res = (out.reshape(nh, nr, d), lse.reshape(nh, nr))
    if with_probs:
        res += (probs.reshape(nh, nr, Sk), probs_hat.reshape(nh, nr, Sk))
    elif with_topk:
        if pct > 0:
            res += (tidx[: nh * nqb * kmax].reshape(nh, nqb, kmax), tcnt[: nh * nqb].reshape(nh, nqb))
        else:
            res += (None, None)
    if tie_slack is not None:
        res += (amb.reshape(nh, nr),)
    return res


def attention_exact(q, k, v, causal=False, softmax_scale=0.0, rows=None, heads=None):
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    ra, nr = _sel(rows, np.int64)
    ha, nh = _sel(heads, np.int32)
    nr = nr if ra is not None else Sq
    nh = nh if ha is not None else B * H
    out = np.zeros(nh * nr * d, np.float32)
    lse = np.zeros(nh * nr, np.float32)
    rc = lib().orc_attention_exact(q.reshape(-1), k.reshape(-1), v.reshape(-1), B, H, Hkv, Sq, Sk, d,
                                   int(causal), float(softmax_scale), _ptr(ra),
                                   nr if ra is not None else 0, _ptr(ha), nh if ha is not None else 0,
                                   out, _ptr(lse))
    if rc != 0:
        raise ValueError("bad attention arguments")
    return out.reshape(nh, nr, d), lse.reshape(nh, nr)


def block_sums(x, blk=128):
    """Binary64 sums over blocks of blk tokens of x [S, d] (ascending tokens)."""
    x = _f32(x)
    S, d = x.shape
    nb = (S + blk - 1) // blk
    out = np.zeros(max(nb * d, 1), np.float64)
    lib().orc_block_sums(x, S, d, blk, out)
    return out[: nb * d].reshape(nb, d)


def attention_decode(q, k, v, ctx_len, n_sink, n_recent, softmax_scale=0.0, scale_search=True,
                     fmin=-2, fmax=6, pairs=None, pct=0, sel_block=128, kmax=None,
                     with_selection=False):
    """Decode oracle. q [B,Hq,d]; k/v [B,Hkv,Lcap,d] original context; ctx_len [B].

    pct > 0 promotes the best ceil(pct * n / 100) middle blocks of sel_block
    tokens per (batch, kv head) to full precision (scored by the mean of the
    group's queries against the block's mean key).  kmax (default: from the
    longest middle) is the row length of the selection output.

    Returns (out [np, G, d], lse [np, G]) for the selected (b*Hkv+kvh) pairs,
    and with with_selection also (sel_idx [np, kmax], sel_cnt [np])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, d = q.shape
    Hkv, Lcap = k.shape[1], k.shape[2]
    G = Hq // Hkv
    cl = np.ascontiguousarray(np.asarray(ctx_len, np.int32).reshape(-1))
    pa, npairs = _sel(pairs, np.int32)
    npairs = npairs if pa is not None else B * Hkv
    out = np.zeros(npairs * G * d, np.float32)
    lse = np.zeros(npairs * G, np.float32)
    if kmax is None:
        mmax = max(int(cl.max()) - n_sink - n_recent, 0)
        kmax = topk_count(pct, (mmax + sel_block - 1) // sel_block) if pct > 0 else 0
    sidx = np.zeros(max(npairs * kmax, 1), np.int32)
    scnt = np.zeros(max(npairs, 1), np.int32)
    rc = lib().orc_attention_decode(q.reshape(-1), k.reshape(-1), v.reshape(-1), cl, B, Hq, Hkv, d,
                                    Lcap, n_sink, n_recent, float(softmax_scale), int(scale_search),
                                    fmin, fmax, _ptr(pa), npairs if pa is not None else 0, out,
                                    _ptr(lse), int(pct), int(sel_block), int(kmax), _ptr(sidx),
                                    _ptr(scnt))
    if rc != 0:
        raise ValueError("bad decode arguments")
    res = (out.reshape(npairs, G, d), lse.reshape(npairs, G))
    if with_selection:
        res += (sidx[: npairs * kmax].reshape(npairs, kmax), scnt[:npairs])
    return res


def kv_append(k_recent, v_recent, k_codes, k_scales, v_codes, v_scales, mid_len, k_new, v_new,
              k_mid=None, v_mid=None, k_sum=None, sel_block=128):
    """Quantize-on-write append (the cache's middle is NVFP4 with ScaleSearch,
    its first and last blocks full precision: ScaleSearch page, Metodologia /
    ScaleSearchAttention).  Steps, per batch b:
      1. T = recent window followed by the new tokens (oldest first);
      2. m = mid_len[b] clamped to [0, mid_cap] and rounded down to a multiple
         of 16; if m + n_new > mid_cap the batch is left unchanged (flag 1);
      3. the first n_new tokens of T are quantized exactly as quantize() does
         for a cache middle region -- K row by row in blocks of 16 channels,
         V in blocks of 16 tokens per channel, ScaleSearch [-2, 6], g = 1 --
         and written at tokens m .. m + n_new;
      4. the window becomes the last n_recent tokens of T; mid_len[b] = m + n_new.
    Arrays are numpy (k/v bf16 values as float32, codes/scales uint8, mid_len
    int32) with the layouts of fp4.h; copies are returned:
    (k_recent, v_recent, k_codes, k_scales, v_codes, v_scales, mid_len, overflow).
    With the full-precision copy of the middle (k_mid, v_mid [B,Hkv,mid_cap,d]
    and the binary64 key-block sums k_sum [B,Hkv,ceil(mid_cap/sel_block),d];
    ThriftAttention page, Significado: both copies kept), step 3 also writes
    the tokens unquantized at m .. m + n_new and adds each one, in order, to
    the sum of its block (a block's sum starts from zero at its first token);
    the three updated copies follow the tuple above."""
    kr, vr = _f32(k_recent).copy(), _f32(v_recent).copy()
    kn, vn = _f32(k_new), _f32(v_new)
    kc, ks = np.array(k_codes, np.uint8), np.array(k_scales, np.uint8)
    vc, vs = np.array(v_codes, np.uint8), np.array(v_scales, np.uint8)
    ml = np.array(mid_len, np.int32).reshape(-1).copy()
    B, Hkv, n_new, d = kn.shape
    n_recent = kr.shape[2]
    mid_cap = kc.shape[2]
    assert n_new % 16 == 0 and n_new > 0
    dual = k_mid is not None
    if dual:
        km, vm = _f32(k_mid).copy(), _f32(v_mid).copy()
        ksum = np.array(k_sum, np.float64)
    over = np.zeros(B, np.int32)
    for b in range(B):
        m = int(min(max(int(ml[b]), 0), mid_cap)) // 16 * 16
        if m + n_new > mid_cap:
            over[b] = 1
            continue
        for h in range(Hkv):
            tk = np.concatenate([kr[b, h], kn[b, h]], axis=0)
            tv = np.concatenate([vr[b, h], vn[b, h]], axis=0)
            if dual:
                km[b, h, m:m + n_new] = tk[:n_new]
                vm[b, h, m:m + n_new] = tv[:n_new]
                for t in range(n_new):
                    j = (m + t) // sel_block
                    if (m + t) % sel_block == 0:
                        ksum[b, h, j] = 0.0
                    ksum[b, h, j] = ksum[b, h, j] + tk[t].astype(np.float64)
            rk = quantize(tk[:n_new], 0, True, -2, 6)
            rv = quantize(tv[:n_new], 1, True, -2, 6)
            kc[b, h, m:m + n_new] = rk["codes"]
            ks[b, h, m:m + n_new] = rk["scales"]
            vc[b, h, m // 2:(m + n_new) // 2] = rv["codes"]
            vs[b, h, m // 16:(m + n_new) // 16] = rv["scales"]
            kr[b, h] = tk[n_new:]
            vr[b, h] = tv[n_new:]
        ml[b] = m + n_new
    if dual:
        return kr, vr, kc, ks, vc, vs, ml, over, km, vm, ksum
    return kr, vr, kc, ks, vc, vs, ml, over


def attention_train(q, k, v, dout, causal=False, softmax_scale=0.0, kv_tile=128, scale_search=True,
                    fmin=-2, fmax=6, single_level_p=False):
    """One training step of FP4 attention with quantization-aware training
    (Attn-QAT page, Metodologia / A and B): the forward of attention_fwd (no
    FP16 path) plus

      O' = P V^, the high-precision output (normalized probabilities P, not
           their FP4 version P^), kept for the backward;
      dV = P^T dO      (P recomputed in FP4, as the forward used it)
      dP = dO V^T
      D  = rowsum(dO * O')   (= rowsum(P * dP): the identity holds for P, not P^)
      dS = s * P * (dP - D)  with s = c ln 2, c the binary32 score factor
      dQ = dS K^,  dK = dS^T Q^  (summed over the query heads of a kv head)

    Q^, K^, V^ are the fake-quantized operands and the quantizers pass the
    gradient straight through (dQ is the gradient of Q^, and so on).  Float64
    throughout.  Returns dict(out, lse, out_hp, dq, dk, dv)."""
    q32, k32, v32 = _f32(q), _f32(k), _f32(v)
    do = _f32(dout).astype(np.float64)
    B, H, Sq, d = q32.shape
    Hkv, Sk = k32.shape[1], k32.shape[2]
    G = H // Hkv
    out, lse, P, Ph = attention_fwd(q32, k32, v32, causal=causal, softmax_scale=softmax_scale, kv_tile=kv_tile,
                                    scale_search=scale_search, fmin=fmin, fmax=fmax,
                                    single_level_p=single_level_p, with_probs=True)
    P = P.reshape(B, H, Sq, Sk)
    Ph = Ph.reshape(B, H, Sq, Sk)
    s = float(score_factor(softmax_scale, d)) * math.log(2.0)

    def fq(x, axis):
        r = quantize(x, axis, scale_search, fmin, fmax)
        return dequantize(r["codes"], r["scales"], x.shape[0], x.shape[1], axis)

    out_hp = np.zeros((B, H, Sq, d))
    dq = np.zeros((B, H, Sq, d))
    dk = np.zeros((B, Hkv, Sk, d))
    dv = np.zeros((B, Hkv, Sk, d))
    for b in range(B):
        kh = [fq(k32[b, j], 0) for j in range(Hkv)]
        vh = [fq(v32[b, j], 1) for j in range(Hkv)]
        for h in range(H):
            j = h // G
            qh = fq(q32[b, h], 0)
            out_hp[b, h] = P[b, h] @ vh[j]
            dv[b, j] += Ph[b, h].T @ do[b, h]
            dP = do[b, h] @ vh[j].T
            D = (do[b, h] * out_hp[b, h]).sum(axis=1)
            dS = s * P[b, h] * (dP - D[:, None])
            dq[b, h] = dS @ kh[j]
            dk[b, j] += dS.T @ qh
    return dict(out=out.reshape(B, H, Sq, d), lse=lse.reshape(B, H, Sq), out_hp=out_hp, dq=dq, dk=dk, dv=dv)
