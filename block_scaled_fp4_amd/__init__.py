"""Block-scaled FP4 (NVFP4-style) attention for AMD MI355X -- Python binding.

Thin ctypes layer over the C ABI in include/fp4.h (libfp4.so, hand-written HIP
kernels for gfx950).  Functions carry the C names and only marshal arguments:
torch tensors provide device memory, torch's current stream is the launch
stream, and every step runs in the library's kernels.  There is no CPU
fallback: without the native library (or a GPU) the calls raise.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "load", "build", "fp4_version", "fp4_last_error", "fp4_quantize", "fp4_block_topk",
    "fp4_attention_fwd", "fp4_attention_decode", "fp4_kv_cache_append", "fp4_kv_block_sums", "decode_sel_kmax",
    "fp4_attention_fwd_train", "fp4_attention_bwd", "fp4_mx_quantize", "fp4_attention_fwd_mx",
    "FP4Error", "BF16", "FP16", "FP32", "GLOBAL_NONE", "GLOBAL_AMAX", "GLOBAL_GIVEN", "KVCache", "lib_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libfp4.so")

BF16, FP16, FP32 = 0, 1, 2
GLOBAL_NONE, GLOBAL_AMAX, GLOBAL_GIVEN = 0, 1, 2
_DT = {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}
_TORCH_DT = {BF16: torch.bfloat16, FP16: torch.float16, FP32: torch.float32}


class FP4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fp4 status {status}: {msg}")
        self.status = status


class QuantOpts(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("scale_search", C.c_int32), ("f_min", C.c_int32),
                ("f_max", C.c_int32), ("global_scale", C.c_int32), ("block_axis", C.c_int32),
                ("hadamard", C.c_int32), ("hadamard_signs", C.c_uint32 * 4), ("channel_exp", C.c_void_p),
                ("exp_negate", C.c_int32), ("exp_rows", C.c_int64)]


class AttnProblem(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("B", C.c_int64), ("H", C.c_int64), ("Hkv", C.c_int64),
                ("Sq", C.c_int64), ("Sk", C.c_int64), ("d", C.c_int64), ("dtype", C.c_int32),
                ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("q_codes", C.c_void_p), ("q_scales", C.c_void_p), ("k_codes", C.c_void_p),
                ("k_scales", C.c_void_p), ("v_codes", C.c_void_p), ("v_scales", C.c_void_p),
                ("q_strides", C.c_int64 * 3), ("k_strides", C.c_int64 * 3), ("v_strides", C.c_int64 * 3)]


class AttnOpts(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("causal", C.c_int32), ("softmax_scale", C.c_float),
                ("kv_tile", C.c_int32), ("scale_search", C.c_int32), ("f_min", C.c_int32),
                ("f_max", C.c_int32), ("fp16_budget_pct", C.c_int32), ("sel_block", C.c_int32),
                ("out_dtype", C.c_int32), ("selection_given", C.c_int32), ("hadamard_qk", C.c_int32),
                ("hadamard_signs", C.c_uint32 * 4), ("p_single_level", C.c_int32), ("balance_qk", C.c_int32)]


def _sign_words(signs):
    """Sign bits of the incoherence rotation as four 32-bit words (None: no flips)."""
    w = (C.c_uint32 * 4)()
    for i, v in enumerate(list(signs or [])[:4]):
        w[i] = int(v) & 0xFFFFFFFF
    return w


class KVCacheStruct(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("B", C.c_int64), ("Hkv", C.c_int64), ("d", C.c_int64),
                ("n_sink", C.c_int32), ("n_recent", C.c_int32), ("mid_cap", C.c_int64),
                ("k_sink", C.c_void_p), ("v_sink", C.c_void_p), ("k_codes", C.c_void_p),
                ("k_scales", C.c_void_p), ("v_codes", C.c_void_p), ("v_scales", C.c_void_p),
                ("k_recent", C.c_void_p), ("v_recent", C.c_void_p), ("mid_len", C.c_void_p),
                ("k_mid", C.c_void_p), ("v_mid", C.c_void_p), ("k_sum", C.c_void_p)]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def build() -> str:
    """Compile libfp4.so for gfx950 (hipcc, in-tree)."""
    from .buildlib import build as _b
    return _b()


def load():
    """Load libfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FP4Error(-4, f"native library missing at {_LIB_PATH}; run block_scaled_fp4_amd.build()")
    L = C.CDLL(_LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    L.fp4_version.restype = C.c_int
    L.fp4_last_error.restype = C.c_char_p
    L.fp4_quantize.argtypes = [vp, i32, i64, i64, i64, C.POINTER(QuantOpts), vp, vp, vp, vp, vp, sz, vp]
    L.fp4_quantize.restype = C.c_int
    L.fp4_quantize_workspace_size.argtypes = [i64, i64, C.POINTER(QuantOpts)]
    L.fp4_quantize_workspace_size.restype = sz
    L.fp4_attention_fwd.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts), vp, vp, vp, vp, vp, sz, vp]
    L.fp4_attention_fwd.restype = C.c_int
    L.fp4_attention_fwd_workspace_size.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts)]
    L.fp4_attention_fwd_workspace_size.restype = sz
    L.fp4_block_topk.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts), vp, vp, vp, sz, vp]
    L.fp4_block_topk.restype = C.c_int
    L.fp4_block_topk_workspace_size.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts)]
    L.fp4_block_topk_workspace_size.restype = sz
    L.fp4_qk_balance.argtypes = [C.POINTER(AttnProblem), vp, vp, sz, vp]
    L.fp4_qk_balance.restype = C.c_int
    L.fp4_qk_balance_workspace_size.argtypes = [C.POINTER(AttnProblem)]
    L.fp4_qk_balance_workspace_size.restype = sz
    L.fp4_attention_decode.argtypes = [vp, i64, C.POINTER(KVCacheStruct), C.c_float, i32, vp, vp, vp, sz, vp]
    L.fp4_attention_decode.restype = C.c_int
    L.fp4_attention_decode_workspace_size.argtypes = [i64, C.POINTER(KVCacheStruct)]
    L.fp4_attention_decode_workspace_size.restype = sz
    L.fp4_attention_decode_noalloc.argtypes = [vp, i64, C.POINTER(KVCacheStruct), C.c_float, i32, vp, vp, vp]
    L.fp4_attention_decode_noalloc.restype = C.c_int
    L.fp4_calib_mfma_f16.argtypes = [i64, i32, vp, vp]
    L.fp4_calib_mfma_f16.restype = C.c_int
    L.fp4_calib_read.argtypes = [vp, sz, i32, vp, vp]
    L.fp4_calib_read.restype = C.c_int
    L.fp4_mx_quantize.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp]
    L.fp4_mx_quantize.restype = C.c_int
    L.fp4_attention_fwd_mx.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts), vp, vp, vp, sz, vp]
    L.fp4_attention_fwd_mx.restype = C.c_int
    L.fp4_attention_fwd_mx_workspace_size.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts)]
    L.fp4_attention_fwd_mx_workspace_size.restype = sz
    L.fp4_attention_fwd_train.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts), vp, vp, vp, vp, sz, vp]
    L.fp4_attention_fwd_train.restype = C.c_int
    L.fp4_attention_bwd.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fp4_attention_bwd.restype = C.c_int
    L.fp4_attention_bwd_workspace_size.argtypes = [C.POINTER(AttnProblem), C.POINTER(AttnOpts)]
    L.fp4_attention_bwd_workspace_size.restype = sz
    L.fp4_attention_decode_selective.argtypes = [vp, i64, C.POINTER(KVCacheStruct), i32, C.c_float, i32, vp, vp,
                                                 vp, vp, vp, sz, vp]
    L.fp4_attention_decode_selective.restype = C.c_int
    L.fp4_attention_decode_selective_workspace_size.argtypes = [i64, C.POINTER(KVCacheStruct), i32]
    L.fp4_attention_decode_selective_workspace_size.restype = sz
    L.fp4_kv_block_sums.argtypes = [C.POINTER(KVCacheStruct), vp]
    L.fp4_kv_block_sums.restype = C.c_int
    L.fp4_kv_cache_append.argtypes = [C.POINTER(KVCacheStruct), vp, vp, i32, vp, vp, sz, vp]
    L.fp4_kv_cache_append.restype = C.c_int
    L.fp4_kv_cache_append_workspace_size.argtypes = [C.POINTER(KVCacheStruct)]
    L.fp4_kv_cache_append_workspace_size.restype = sz
    _lib = L
    return L


def fp4_version() -> int:
    return load().fp4_version()


def fp4_last_error() -> str:
    return load().fp4_last_error().decode()


def _check(st: int):
    if st != 0:
        raise FP4Error(st, fp4_last_error())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise FP4Error(-1, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise FP4Error(-1, f"{name} must be contiguous")


def _dev_rows(t, name):
    """A 4-D attention input [B, heads, S, d]: a GPU tensor whose rows of d
    elements are contiguous (other strides are passed to the library)."""
    if t is None:
        return
    if not t.is_cuda:
        raise FP4Error(-1, f"{name} must be a GPU tensor")
    if t.dim() != 4 or t.stride(-1) != 1:
        raise FP4Error(-1, f"{name} must be 4-D with contiguous rows (last stride 1)")


def _strides(t):
    """{batch, head, token} element strides of a 4-D input, or zeros when it
    is dense (the library's default).  Strides of size-1 dimensions never
    multiply a non-zero index; they are normalized so the library's checks see
    whole rows."""
    w = (C.c_int64 * 3)()
    if t is None or t.is_contiguous():
        return w
    B, Hn, S, d = t.shape
    sb, sh, ss, _ = t.stride()
    w[0] = 0 if B == 1 else sb
    w[1] = 0 if Hn == 1 else sh
    w[2] = d if S == 1 else ss
    return w


def _out(out, shape, dtype, dev, name="out"):
    """The output buffer: allocated when not given; a given one must be a
    contiguous GPU tensor of exactly the dtype and element count the kernel
    writes (the C ABI takes a bare pointer and cannot check)."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _dev(out, name)
    n = 1
    for x in shape:
        n *= int(x)
    if out.dtype != dtype or out.numel() != n:
        raise FP4Error(-1, f"{name} must be {dtype} with {n} elements (got {out.dtype}, {out.numel()})")
    return out


def _stream(dev):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(n, dev):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev) if n else None


def fp4_quantize(x: torch.Tensor, block_axis: int = 0, scale_search: bool = True, f_min: int = -2,
                 f_max: int = 6, global_scale: int = GLOBAL_NONE, g: torch.Tensor | None = None,
                 with_offsets: bool = True, out=None, hadamard: bool = False, hadamard_signs=None,
                 channel_exp=None, exp_negate: bool = False, exp_rows: int = 1):
    """Quantize a 2-D tensor (bf16/fp16/fp32, contiguous rows) to NVFP4 blocks.

    hadamard rotates each row first (incoherence processing; hadamard_signs:
    up to four 32-bit words of sign bits).  channel_exp (int32 GPU tensor
    [rows / exp_rows, cols], e.g. from fp4_qk_balance) first multiplies row r
    by 2^(+-e[r // exp_rows]) (minus with exp_negate).  Returns dict(codes,
    scales, offsets, g); layouts as documented in fp4.h."""
    L = load()
    _dev(x, "x")
    rows, cols = x.shape
    dev = x.device
    if block_axis == 0:
        cshape, sshape = (rows, cols // 2), (rows, cols // 16)
    else:
        cshape, sshape = (rows // 2, cols), (rows // 16, cols)
    if out is not None:
        codes = _out(out["codes"], cshape, torch.uint8, dev, "codes")
        scales = _out(out["scales"], sshape, torch.uint8, dev, "scales")
        offs = out.get("offsets")
        offs = _out(offs, sshape, torch.int8, dev, "offsets") if offs is not None else None
    else:
        codes = torch.empty(cshape, dtype=torch.uint8, device=dev)
        scales = torch.empty(sshape, dtype=torch.uint8, device=dev)
        offs = torch.empty(sshape, dtype=torch.int8, device=dev) if with_offsets else None
    if g is None and global_scale != GLOBAL_NONE:
        g = torch.empty(1, dtype=torch.float32, device=dev)
    if channel_exp is not None:
        _dev(channel_exp, "channel_exp")
        if channel_exp.dtype != torch.int32 or channel_exp.numel() * int(exp_rows) != rows * cols:
            raise FP4Error(-1, "channel_exp must be int32 with rows / exp_rows * cols elements")
    o = QuantOpts(C.sizeof(QuantOpts), int(bool(scale_search)), f_min, f_max, global_scale, block_axis,
                  int(bool(hadamard)), _sign_words(hadamard_signs), _ptr(channel_exp), int(bool(exp_negate)),
                  int(exp_rows))
    nws = L.fp4_quantize_workspace_size(rows, cols, C.byref(o))
    ws = _workspace(nws, dev)
    st = L.fp4_quantize(_ptr(x), _DT[x.dtype], rows, cols, cols, C.byref(o), _ptr(codes), _ptr(scales),
                        _ptr(offs), _ptr(g), _ptr(ws), nws, _stream(dev))
    _check(st)
    return dict(codes=codes, scales=scales, offsets=offs, g=g)


def fp4_mx_quantize(x: torch.Tensor, block_axis: int = 0):
    """MXFP4 quantization of a 2-D tensor (blocks of 32, E8M0 scales).
    Returns dict(codes, scales)."""
    L = load()
    _dev(x, "x")
    rows, cols = x.shape
    dev = x.device
    if block_axis == 0:
        cshape, sshape = (rows, cols // 2), (rows, cols // 32)
    else:
        cshape, sshape = (rows // 2, cols), (rows // 32, cols)
    codes = torch.empty(cshape, dtype=torch.uint8, device=dev)
    scales = torch.empty(sshape, dtype=torch.uint8, device=dev)
    _check(L.fp4_mx_quantize(_ptr(x), _DT[x.dtype], rows, cols, cols, block_axis, _ptr(codes), _ptr(scales),
                             _stream(dev)))
    return dict(codes=codes, scales=scales)


def _problem(q, k, v, quant=None):
    B, H, Sq, d = q.shape if q is not None else quant["q_shape"]
    Hkv, Sk = (k.shape[1], k.shape[2]) if k is not None else quant["kv_shape"]
    dt = _DT[q.dtype] if q is not None else BF16
    P = AttnProblem(C.sizeof(AttnProblem), B, H, Hkv, Sq, Sk, d, dt, _ptr(q), _ptr(k), _ptr(v))
    P.q_strides, P.k_strides, P.v_strides = _strides(q), _strides(k), _strides(v)
    if quant is not None:
        for name in ("q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"):
            setattr(P, name, _ptr(quant[name]))
    return P


def _opts(causal, softmax_scale, kv_tile, scale_search, f_min, f_max, pct, sel_block, out_dtype, given=False,
          hadamard=False, hadamard_signs=None, single_level_p=False, balance=False):
    return AttnOpts(C.sizeof(AttnOpts), int(bool(causal)), float(softmax_scale), kv_tile,
                    int(bool(scale_search)), f_min, f_max, int(pct), sel_block, out_dtype, int(bool(given)),
                    int(bool(hadamard)), _sign_words(hadamard_signs), int(bool(single_level_p)), int(bool(balance)))


def fp4_qk_balance(q, k):
    """Exponents e [B, Hkv, d] (int32) of the balance pair Q 2^-e, K 2^e
    (fp4.h: fp4_qk_balance).  q [B,H,Sq,d], k [B,Hkv,Sk,d] bf16 or fp16."""
    L = load()
    for t, n in ((q, "q"), (k, "k")):
        _dev_rows(t, n)
    P = _problem(q, k, k)
    B, Hkv, d = k.shape[0], k.shape[1], k.shape[3]
    e = torch.empty((B, Hkv, d), dtype=torch.int32, device=q.device)
    nws = L.fp4_qk_balance_workspace_size(C.byref(P))
    ws = _workspace(nws, q.device)
    _check(L.fp4_qk_balance(C.byref(P), _ptr(e), _ptr(ws), nws, _stream(q.device)))
    return e


def fp4_block_topk(q, k, causal=True, fp16_budget_pct=10, sel_block=128, kv_tile=128):
    """Block selection alone: returns (idx [B,H,nqb,kmax], cnt [B,H,nqb])."""
    L = load()
    for t, n in ((q, "q"), (k, "k")):
        _dev_rows(t, n)
    P = _problem(q, k, k)
    O = _opts(causal, 0.0, kv_tile, True, -2, 6, fp16_budget_pct, sel_block, FP32)
    B, H, Sq = q.shape[:3]
    Sk = k.shape[2]
    nqb = (Sq + sel_block - 1) // sel_block
    nkb = (Sk + sel_block - 1) // sel_block
    kmax = (fp16_budget_pct * nkb + 99) // 100
    idx = torch.empty((B, H, nqb, max(kmax, 1)), dtype=torch.int32, device=q.device)
    cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=q.device)
    nws = L.fp4_block_topk_workspace_size(C.byref(P), C.byref(O))
    ws = _workspace(nws, q.device)
    _check(L.fp4_block_topk(C.byref(P), C.byref(O), _ptr(idx), _ptr(cnt), _ptr(ws), nws, _stream(q.device)))
    return idx[..., :kmax], cnt


def fp4_attention_fwd(q, k, v, causal=False, softmax_scale=0.0, kv_tile=128, scale_search=True, f_min=-2,
                      f_max=6, fp16_budget_pct=0, sel_block=128, out_dtype=BF16, quantized=None,
                      return_lse=True, return_topk=False, workspace=None, out=None, selection=None,
                      hadamard=False, hadamard_signs=None, single_level_p=False, balance=False):
    """FP4 attention forward.  q [B,H,Sq,d], k/v [B,Hkv,Sk,d] (bf16 or fp16).

    single_level_p: P is quantized with the NVFP4 block scale alone (no row
    level).

    hadamard: Q and K are quantized after the incoherence rotation (with
    hadamard_signs); the scores are unchanged in exact arithmetic.

    quantized: optional dict with q_codes..v_scales from fp4_quantize (then q/k/v
    may be None when fp16_budget_pct == 0).  selection: optional (idx, cnt) from
    fp4_block_topk, used instead of computing one.  Returns (out, lse[, idx, cnt])."""
    L = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_rows(t, n)
    ref = q if q is not None else quantized["q_codes"]
    dev = ref.device
    if q is not None:
        B, H, Sq, d = q.shape
    else:
        B, H, Sq, d = quantized["q_shape"]
    P = _problem(q, k, v, quantized)
    O = _opts(causal, softmax_scale, kv_tile, scale_search, f_min, f_max, fp16_budget_pct, sel_block, out_dtype,
              selection is not None, hadamard, hadamard_signs, single_level_p, balance)
    out = _out(out, (B, H, Sq, d), _TORCH_DT[out_dtype], dev)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev) if return_lse else None
    idx = cnt = None
    if selection is not None:
        idx, cnt = selection
        _dev(idx, "selection idx")
        _dev(cnt, "selection cnt")
    elif return_topk and fp16_budget_pct > 0:
        Sk = P.Sk
        nqb = (Sq + sel_block - 1) // sel_block
        nkb = (Sk + sel_block - 1) // sel_block
        kmax = (fp16_budget_pct * nkb + 99) // 100
        idx = torch.empty((B, H, nqb, kmax), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, H, nqb), dtype=torch.int32, device=dev)
    nws = L.fp4_attention_fwd_workspace_size(C.byref(P), C.byref(O))
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, dev)
    _check(L.fp4_attention_fwd(C.byref(P), C.byref(O), _ptr(out), _ptr(lse), _ptr(idx), _ptr(cnt), _ptr(ws),
                               nws, _stream(dev)))
    return (out, lse, idx, cnt) if return_topk else (out, lse)


def fp4_attention_fwd_mx(q, k, v, causal=False, softmax_scale=0.0, kv_tile=128, out_dtype=BF16, quantized=None,
                         return_lse=True, workspace=None, out=None):
    """MXFP4 attention forward (blocks of 32, power-of-two scales, P quantized
    per 32 keys against the tile reference ceil(max x)).  q [B,H,Sq,d], k/v
    [B,Hkv,Sk,d]; quantized: optional dict with q_codes..v_scales from
    fp4_mx_quantize plus q_shape/kv_shape.  Returns (out, lse)."""
    L = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_rows(t, n)  # (the library rejects strided inputs here)
    ref = q if q is not None else quantized["q_codes"]
    dev = ref.device
    B, H, Sq, d = q.shape if q is not None else quantized["q_shape"]
    P = _problem(q, k, v, quantized)
    O = _opts(causal, softmax_scale, kv_tile, False, -2, 6, 0, 128, out_dtype, False)
    out = _out(out, (B, H, Sq, d), _TORCH_DT[out_dtype], dev)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev) if return_lse else None
    nws = L.fp4_attention_fwd_mx_workspace_size(C.byref(P), C.byref(O))
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, dev)
    _check(L.fp4_attention_fwd_mx(C.byref(P), C.byref(O), _ptr(out), _ptr(lse), _ptr(ws), nws, _stream(dev)))
    return out, lse


def fp4_attention_fwd_train(q, k, v, causal=False, softmax_scale=0.0, kv_tile=128, scale_search=True, f_min=-2,
                            f_max=6, out_dtype=FP32, single_level_p=False, workspace=None):
    """Training forward: (out, out_hp, lse) -- out and lse as fp4_attention_fwd,
    out_hp the high-precision output O' kept for the backward."""
    L = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_rows(t, n)
    B, H, Sq, d = q.shape
    P = _problem(q, k, v)
    O = _opts(causal, softmax_scale, kv_tile, scale_search, f_min, f_max, 0, 128, out_dtype,
              single_level_p=single_level_p)
    out = torch.empty((B, H, Sq, d), dtype=_TORCH_DT[out_dtype], device=q.device)
    out_hp = torch.empty_like(out)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    nws = L.fp4_attention_fwd_workspace_size(C.byref(P), C.byref(O))
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, q.device)
    _check(L.fp4_attention_fwd_train(C.byref(P), C.byref(O), _ptr(out), _ptr(out_hp), _ptr(lse), _ptr(ws), nws,
                                     _stream(q.device)))
    return out, out_hp, lse


def fp4_attention_bwd(q, k, v, out_hp, lse, dout, causal=False, softmax_scale=0.0, kv_tile=128, scale_search=True,
                      f_min=-2, f_max=6, single_level_p=False, workspace=None):
    """Training backward: (dq, dk, dv) in float32 from fp4_attention_fwd_train's
    out_hp and lse and the output gradient dout (q's dtype)."""
    L = load()
    for t, n in ((out_hp, "out_hp"), (lse, "lse"), (dout, "dout")):
        _dev(t, n)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_rows(t, n)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    hp_dtype = {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}[out_hp.dtype]
    P = _problem(q, k, v)
    O = _opts(causal, softmax_scale, kv_tile, scale_search, f_min, f_max, 0, 128, hp_dtype,
              single_level_p=single_level_p)
    dq = torch.empty((B, H, Sq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, Sk, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, Sk, d), dtype=torch.float32, device=q.device)
    nws = L.fp4_attention_bwd_workspace_size(C.byref(P), C.byref(O))
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, q.device)
    _check(L.fp4_attention_bwd(C.byref(P), C.byref(O), _ptr(out_hp), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(ws), nws, _stream(q.device)))
    return dq, dk, dv


def attention_fwd_workspace_bytes(q_shape, kv_shape, causal=False, kv_tile=128, fp16_budget_pct=0,
                                  sel_block=128, prequantized=False):
    L = load()
    B, H, Sq, d = q_shape
    Hkv, Sk = kv_shape
    P = AttnProblem(C.sizeof(AttnProblem), B, H, Hkv, Sq, Sk, d, BF16)
    if prequantized:
        for name in ("q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"):
            setattr(P, name, C.c_void_p(16))
    O = _opts(causal, 0.0, kv_tile, True, -2, 6, fp16_budget_pct, sel_block, BF16)
    return L.fp4_attention_fwd_workspace_size(C.byref(P), C.byref(O))


class KVCache:
    """Device buffers of a sink-aware mixed-precision KV cache (layouts in fp4.h).

    k_mid, v_mid (bf16 [B,Hkv,mid_cap,d]) and k_sum (float64
    [B,Hkv,ceil(mid_cap/128),d]) are the optional full-precision copy of the
    middle that selective decode reads."""

    def __init__(self, k_sink, v_sink, k_codes, k_scales, v_codes, v_scales, k_recent, v_recent, mid_len,
                 k_mid=None, v_mid=None, k_sum=None):
        self.k_mid, self.v_mid, self.k_sum = k_mid, v_mid, k_sum
        self.k_sink, self.v_sink = k_sink, v_sink
        self.k_codes, self.k_scales, self.v_codes, self.v_scales = k_codes, k_scales, v_codes, v_scales
        self.k_recent, self.v_recent = k_recent, v_recent
        self.mid_len = mid_len
        self.B, self.Hkv = k_codes.shape[0], k_codes.shape[1]
        self.d = k_codes.shape[3] * 2
        self.mid_cap = k_codes.shape[2]
        self.n_sink = k_sink.shape[2]
        self.n_recent = k_recent.shape[2]

    def struct(self):
        return KVCacheStruct(C.sizeof(KVCacheStruct), self.B, self.Hkv, self.d, self.n_sink, self.n_recent,
                             self.mid_cap, _ptr(self.k_sink), _ptr(self.v_sink), _ptr(self.k_codes),
                             _ptr(self.k_scales), _ptr(self.v_codes), _ptr(self.v_scales), _ptr(self.k_recent),
                             _ptr(self.v_recent), _ptr(self.mid_len), _ptr(self.k_mid), _ptr(self.v_mid),
                             _ptr(self.k_sum))


def decode_sel_kmax(mid_cap, fp16_budget_pct):
    """Row length of the selective decode's selection output."""
    nbc = (mid_cap + 127) // 128
    return (fp16_budget_pct * nbc + 99) // 100


def fp4_attention_decode(q, cache: KVCache, softmax_scale=0.0, out_dtype=BF16, return_lse=True, workspace=None,
                         out=None, fp16_budget_pct=0, return_selection=False):
    """One-token decode.  q [B,Hq,d] bf16.  Returns (out [B,Hq,d], lse [B,Hq]),
    and with return_selection also (sel_idx [B,Hkv,kmax], sel_cnt [B,Hkv]).
    fp16_budget_pct > 0 runs the selective decode (needs the cache's
    full-precision copy)."""
    L = load()
    _dev(q, "q")
    B, Hq, d = q.shape
    cs = cache.struct()
    out = _out(out, (B, Hq, d), _TORCH_DT[out_dtype], q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    pct = int(fp16_budget_pct)
    sidx = scnt = None
    if return_selection:
        kmax = decode_sel_kmax(cache.mid_cap, pct) if pct > 0 else 0
        sidx = torch.empty((cache.B, cache.Hkv, kmax), dtype=torch.int32, device=q.device)
        scnt = torch.zeros((cache.B, cache.Hkv), dtype=torch.int32, device=q.device)
    if pct == 0:
        nws = L.fp4_attention_decode_workspace_size(Hq, C.byref(cs))
        ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, q.device)
        _check(L.fp4_attention_decode(_ptr(q), Hq, C.byref(cs), float(softmax_scale), out_dtype, _ptr(out),
                                      _ptr(lse), _ptr(ws), nws, _stream(q.device)))
    else:
        nws = L.fp4_attention_decode_selective_workspace_size(Hq, C.byref(cs), pct)
        ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, q.device)
        _check(L.fp4_attention_decode_selective(_ptr(q), Hq, C.byref(cs), pct, float(softmax_scale), out_dtype,
                                                _ptr(out), _ptr(lse), _ptr(sidx if sidx is not None and sidx.numel() else None),
                                                _ptr(scnt), _ptr(ws), nws, _stream(q.device)))
    if return_selection:
        return out, lse, sidx, scnt
    return out, lse


def fp4_attention_decode_noalloc(q, cache: KVCache, softmax_scale=0.0, out_dtype=BF16, out=None, lse=None):
    """fp4_attention_decode with the library's fixed device scratch array as
    its workspace (no allocation inside the call).  q [B,Hq,d] bf16; out
    [B,Hq,d] and lse [B,Hq] (float32, optional) are the caller's (allocated
    here only when not given).  Returns (out, lse)."""
    L = load()
    _dev(q, "q")
    B, Hq, d = q.shape
    cs = cache.struct()
    out = _out(out, (B, Hq, d), _TORCH_DT[out_dtype], q.device)
    lse = _out(lse, (B, Hq), torch.float32, q.device, "lse") if lse is not None else None
    _check(L.fp4_attention_decode_noalloc(_ptr(q), Hq, C.byref(cs), float(softmax_scale), out_dtype, _ptr(out),
                                          _ptr(lse), _stream(q.device)))
    return out, lse


def fp4_kv_block_sums(cache: KVCache):
    """(Re)compute cache.k_sum from cache.k_mid over the tokens in use."""
    L = load()
    cs = cache.struct()
    dev = cache.k_mid.device if cache.k_mid is not None else torch.device("cuda")
    _check(L.fp4_kv_block_sums(C.byref(cs), _stream(dev)))


def fp4_kv_cache_append(cache: KVCache, k_new, v_new, workspace=None):
    """Quantize-on-write: append k_new, v_new (bf16 [B,Hkv,n_new,d], n_new a
    multiple of 16) to the cache in place.  Returns overflow [B] int32 (1 where
    the NVFP4 region had no room and the batch was left unchanged)."""
    L = load()
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    n_new = int(k_new.shape[2])
    cs = cache.struct()
    overflow = torch.empty((cache.B,), dtype=torch.int32, device=k_new.device)
    nws = L.fp4_kv_cache_append_workspace_size(C.byref(cs))
    ws = workspace if workspace is not None and workspace.numel() >= nws else _workspace(nws, k_new.device)
    _check(L.fp4_kv_cache_append(C.byref(cs), _ptr(k_new), _ptr(v_new), n_new, _ptr(overflow), _ptr(ws), nws,
                                 _stream(k_new.device)))
    return overflow


def calib_mfma_f16(iters: int, workgroups: int, sink):
    """Measurement helper (fp4_calib.h): `workgroups` x 4 waves of four
    independent fp16 32x32x16 MFMA chains, `iters` rounds each.  sink: float32
    GPU tensor of workgroups * 256 elements."""
    L = load()
    _out(sink, (workgroups * 256,), torch.float32, sink.device, "sink")
    st = L.fp4_calib_mfma_f16(int(iters), int(workgroups), _ptr(sink), _stream(sink.device))
    if st != 0:
        raise FP4Error(st, "fp4_calib_mfma_f16 failed")


def calib_read(buf, workgroups: int, sink):
    """Measurement helper (fp4_calib.h): read buf (a contiguous GPU tensor,
    byte size a multiple of 16) once.  sink: int32 GPU tensor of workgroups * 256."""
    L = load()
    _dev(buf, "buf")
    _out(sink, (workgroups * 256,), torch.int32, sink.device, "sink")
    st = L.fp4_calib_read(_ptr(buf), buf.numel() * buf.element_size(), int(workgroups), _ptr(sink),
                          _stream(buf.device))
    if st != 0:
        raise FP4Error(st, "fp4_calib_read failed")

