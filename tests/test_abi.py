"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fp4.h declares, and rejects invalid arguments before launching anything."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared():
    """Every function declared by a header under include/."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(fp4_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    import block_scaled_fp4_amd as fp4
    if not os.path.exists(fp4.lib_path()):
        fp4.build()
    return fp4.load()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"fp4_quantize", "fp4_attention_fwd", "fp4_attention_decode", "fp4_block_topk",
            "fp4_calib_mfma_f16", "fp4_calib_read"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.fp4_version() == 10000


def test_quantize_rejects_bad_arguments(L):
    import block_scaled_fp4_amd as fp4
    opts = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 0, 0)
    fake = C.c_void_p(1 << 20)  # never dereferenced: validation fails first
    st = L.fp4_quantize(fake, 0, 16, 40, 40, C.byref(opts), fake, fake, None, None, None, 0, None)
    assert st == -1 and "cols" in L.fp4_last_error().decode()
    st = L.fp4_quantize(fake, 7, 16, 32, 32, C.byref(opts), fake, fake, None, None, None, 0, None)
    assert st == -1
    bad = fp4.QuantOpts(4, 1, -2, 6, 0, 0)
    assert L.fp4_quantize(fake, 0, 16, 32, 32, C.byref(bad), fake, fake, None, None, None, 0, None) == -1
    rng = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, 1, 6, 0, 0)
    assert L.fp4_quantize(fake, 0, 16, 32, 32, C.byref(rng), fake, fake, None, None, None, 0, None) == -1
    ax1 = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 0, 1)
    assert L.fp4_quantize(fake, 0, 20, 32, 32, C.byref(ax1), fake, fake, None, None, None, 0, None) == -1
    amax = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 1, 0)
    need = L.fp4_quantize_workspace_size(64, 128, C.byref(amax))
    assert need > 0
    st = L.fp4_quantize(fake, 0, 64, 128, 128, C.byref(amax), fake, fake, None, fake, fake, need - 1, None)
    assert st == -3
    st = L.fp4_quantize(fake, 0, 64, 128, 128, C.byref(amax), fake, fake, None, None, fake, need, None)
    assert st == -1  # g required
    mis = C.c_void_p((1 << 20) + 2)
    assert L.fp4_quantize(mis, 0, 16, 32, 32, C.byref(opts), fake, fake, None, None, None, 0, None) == -1


def _prob(fp4, **kw):
    f = C.c_void_p(1 << 20)
    P = fp4.AttnProblem(C.sizeof(fp4.AttnProblem), 1, 2, 2, 256, 256, 128, 0, f, f, f)
    for k, v in kw.items():
        setattr(P, k, v)
    return P


def _opts(fp4, **kw):
    O = fp4.AttnOpts(C.sizeof(fp4.AttnOpts), 1, 0.0, 128, 1, -2, 6, 0, 128, 2)
    for k, v in kw.items():
        setattr(O, k, v)
    return O


def test_attention_rejects_bad_arguments(L):
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)

    def call(P, O, ws_bytes=1 << 40):
        return L.fp4_attention_fwd(C.byref(P), C.byref(O), f, None, None, None, f, ws_bytes, None)

    assert call(_prob(fp4, d=96), _opts(fp4)) == -2
    assert call(_prob(fp4, Sk=250, Sq=250), _opts(fp4)) == -1
    assert call(_prob(fp4, Sq=128), _opts(fp4)) == -1            # causal needs Sq == Sk
    assert call(_prob(fp4, H=3, Hkv=2), _opts(fp4)) == -1
    assert call(_prob(fp4), _opts(fp4, kv_tile=32)) == -2
    assert call(_prob(fp4), _opts(fp4, fp16_budget_pct=101)) == -1
    assert call(_prob(fp4), _opts(fp4, fp16_budget_pct=10, sel_block=192)) == -1
    assert call(_prob(fp4), _opts(fp4, fp16_budget_pct=10, sel_block=64, kv_tile=64)) == -1
    assert call(_prob(fp4, dtype=2), _opts(fp4)) == -2
    assert call(_prob(fp4, q_codes=f), _opts(fp4)) == -1          # partial quantized set
    assert call(_prob(fp4), _opts(fp4), ws_bytes=0) == -3
    assert L.fp4_attention_fwd(None, None, f, None, None, None, f, 0, None) == -1
    assert L.fp4_block_topk(C.byref(_prob(fp4)), C.byref(_opts(fp4)), f, f, f, 1 << 30, None) == -1  # pct 0


def test_decode_rejects_bad_arguments(L):
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)
    cs = fp4.KVCacheStruct(C.sizeof(fp4.KVCacheStruct), 2, 2, 128, 16, 32, 100, f, f, f, f, f, f, f, f, f)
    assert L.fp4_attention_decode(f, 8, C.byref(cs), 0.0, 2, f, None, f, 1 << 30, None) == -1  # mid_cap % 16
    cs.mid_cap = 96
    assert L.fp4_attention_decode(f, 7, C.byref(cs), 0.0, 2, f, None, f, 1 << 30, None) == -1  # Hq % Hkv
    assert L.fp4_attention_decode(f, 64, C.byref(cs), 0.0, 2, f, None, f, 1 << 30, None) == -2  # G > 16
    cs.d = 80
    assert L.fp4_attention_decode(f, 8, C.byref(cs), 0.0, 2, f, None, f, 1 << 30, None) == -2
    cs.d = 128
    need = L.fp4_attention_decode_workspace_size(8, C.byref(cs))
    assert need > 0
    assert L.fp4_attention_decode(f, 8, C.byref(cs), 0.0, 2, f, None, f, need - 1, None) == -3


def test_kv_append_rejects_bad_arguments(L):
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)
    cs = fp4.KVCacheStruct(C.sizeof(fp4.KVCacheStruct), 2, 2, 128, 16, 32, 96, f, f, f, f, f, f, f, f, f)
    need = L.fp4_kv_cache_append_workspace_size(C.byref(cs))
    assert need >= 2 * 2 * 2 * 32 * 128 * 2  # two window copies (K, V) in bf16
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 24, None, f, need, None) == -1   # not a multiple of 16
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 0, None, f, need, None) == -1
    assert L.fp4_kv_cache_append(C.byref(cs), None, f, 16, None, f, need, None) == -1
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 16, None, f, need - 1, None) == -3
    cs.mid_cap = 100
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 16, None, f, need, None) == -1  # capacity % 16
    cs.mid_cap = 96
    cs.d = 96
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 16, None, f, need, None) == -2
    cs.d = 128
    cs.mid_len = None
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 16, None, f, need, None) == -1


def test_selective_decode_and_block_sums_reject_bad_arguments(L):
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)
    cs = fp4.KVCacheStruct(C.sizeof(fp4.KVCacheStruct), 2, 2, 128, 16, 32, 256, f, f, f, f, f, f, f, f, f,
                           f, f, f)
    base = L.fp4_attention_decode_workspace_size(8, C.byref(cs))
    need = L.fp4_attention_decode_selective_workspace_size(8, C.byref(cs), 10)
    assert need > base > 0  # selection keys, indices, counts and mask on top of the partials
    assert L.fp4_attention_decode_selective_workspace_size(8, C.byref(cs), 101) == 0
    assert L.fp4_attention_decode_selective_workspace_size(8, C.byref(cs), 0) == base

    def call(pct, nbytes=need):
        return L.fp4_attention_decode_selective(f, 8, C.byref(cs), pct, 0.0, 2, f, None, None, None, f, nbytes, None)

    assert call(-1) == -1 and call(101) == -1
    assert call(10, need - 1) == -3
    cs.k_sum = None
    assert call(10) == -1  # the budget needs the full-precision copy
    assert L.fp4_kv_block_sums(C.byref(cs), None) == -1
    cs.k_sum = C.c_void_p((1 << 20) + 8)
    assert call(10) == -1  # 16-byte alignment
    assert L.fp4_kv_block_sums(C.byref(cs), None) == -1
    cs.k_sum = f
    cs.mid_cap = 100
    assert L.fp4_kv_block_sums(C.byref(cs), None) == -1
    cs.mid_cap = 256
    cs.d = 96
    assert L.fp4_kv_block_sums(C.byref(cs), None) == -2
    cs.d = 128
    cs.v_mid = None
    assert L.fp4_kv_cache_append(C.byref(cs), f, f, 16, None, f, 1 << 30, None) == -1  # all three or none


def test_hadamard_options_are_validated(L):
    import block_scaled_fp4_amd as fp4
    fake = C.c_void_p(1 << 20)

    def q(cols, axis=0, gmode=0, had=1, rows=32):
        o = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, gmode, axis, had)
        return L.fp4_quantize(fake, 0, rows, cols, cols, C.byref(o), fake, fake, None, fake, fake, 1 << 20, None)

    assert q(128, axis=1) == -1          # rows of blocks only
    assert q(48) == -2                   # not a power of two
    assert q(256) == -2                  # wider than one 8-lane row group
    assert q(128, gmode=1) == -1         # amax of the rotated tensor is not formed
    assert q(128, had=2) == -1
    f = C.c_void_p(1 << 20)

    def call(P, O):
        return L.fp4_attention_fwd(C.byref(P), C.byref(O), f, None, None, None, f, 1 << 40, None)

    quant = dict(q_codes=f, q_scales=f, k_codes=f, k_scales=f, v_codes=f, v_scales=f)
    assert call(_prob(fp4, **quant), _opts(fp4, hadamard_qk=1)) == -1
    assert call(_prob(fp4), _opts(fp4, hadamard_qk=3)) == -1


def test_mx_entry_points_validate(L):
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)
    assert L.fp4_mx_quantize(f, 0, 16, 48, 48, 0, f, f, None) == -1      # cols % 32
    assert L.fp4_mx_quantize(f, 0, 48, 32, 32, 1, f, f, None) == -1      # rows % 32 along rows
    assert L.fp4_mx_quantize(f, 5, 32, 32, 32, 0, f, f, None) == -1      # dtype
    assert L.fp4_mx_quantize(f, 0, 32, 32, 32, 2, f, f, None) == -1      # axis
    assert L.fp4_mx_quantize(C.c_void_p((1 << 20) + 4), 0, 32, 32, 32, 0, f, f, None) == -1

    def call(P, O, ws=1 << 40):
        return L.fp4_attention_fwd_mx(C.byref(P), C.byref(O), f, None, f, ws, None)

    assert call(_prob(fp4, Sq=272, Sk=272), _opts(fp4)) == -1                  # Sk % 32
    assert call(_prob(fp4), _opts(fp4, fp16_budget_pct=10)) == -1              # no FP16 path
    assert call(_prob(fp4), _opts(fp4, hadamard_qk=1)) == -1
    assert call(_prob(fp4, d=96), _opts(fp4)) == -2
    need = L.fp4_attention_fwd_mx_workspace_size(C.byref(_prob(fp4)), C.byref(_opts(fp4)))
    nq = 2 * 256 * 128
    assert need >= nq // 2 + nq // 32 + 2 * (nq // 2 + nq // 32)
    assert call(_prob(fp4), _opts(fp4), need - 1) == -3
    quant = dict(q_codes=f, q_scales=f, k_codes=f, k_scales=f, v_codes=f, v_scales=f)
    assert L.fp4_attention_fwd_mx_workspace_size(C.byref(_prob(fp4, **quant)), C.byref(_opts(fp4))) == 0


def test_log_switch_reports_errors(L, capfd, monkeypatch):
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)
    opts = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 0, 0)
    monkeypatch.setenv("FP4_LOG", "1")
    assert L.fp4_quantize(f, 0, 16, 40, 40, C.byref(opts), f, f, None, None, None, 0, None) == -1
    err = capfd.readouterr().err
    assert "[fp4] error -1" in err and "cols" in err
    monkeypatch.setenv("FP4_LOG", "0")
    assert L.fp4_quantize(f, 0, 16, 40, 40, C.byref(opts), f, f, None, None, None, 0, None) == -1
    assert "[fp4]" not in capfd.readouterr().err


def test_backward_rejects_query_rows_past_32_bit_offsets(L):
    """The dK/dV kernels address one head's query rows through 32-bit buffer
    offsets: Sq * d * 2 must stay below 2^31 (as Sk * d does for every call)."""
    import block_scaled_fp4_amd as fp4
    f = C.c_void_p(1 << 20)

    def call(P):  # no workspace: a call past every other check stops there, before any launch
        return L.fp4_attention_bwd(C.byref(P), C.byref(_opts(fp4, causal=0)), f, f, f, f, f, f, f, 0, None)

    assert call(_prob(fp4, Sq=1 << 23, Sk=256)) == -2          # 2^23 * 128 * 2 = 2^31
    assert call(_prob(fp4, Sq=(1 << 23) - 16, Sk=256)) == -3   # below the limit: the workspace check


def test_backward_workspace_is_linear_in_length(L):
    """The backward recomputes the scores: its workspace holds per-row operand copies only."""
    import block_scaled_fp4_amd as fp4
    sizes = []
    for S in (4096, 8192, 131072):
        P = _prob(fp4, Sq=S, Sk=S, H=32, Hkv=32)
        sizes.append(L.fp4_attention_bwd_workspace_size(C.byref(P), C.byref(_opts(fp4))))
    assert sizes[1] <= 2 * sizes[0] + 4096
    assert sizes[2] <= 32 * sizes[0] + 65536
    n = 32 * 131072 * 128
    # bf16 copies of Q^, K^, V^ and the two terms of an fp16 dO, the row term D, and the NVFP4
    # codes + scales of Q, K, V
    assert sizes[2] < 5 * n * 2 + 32 * 131072 * 4 + 3 * n * 9 // 16 + 65536


def test_noalloc_decode_rejects_oversized_problems(L):
    """The allocation-free decode refuses a problem whose workspace exceeds its
    fixed array, before touching the device, with a message naming the sizes."""
    import block_scaled_fp4_amd as fp4
    cs = fp4.KVCacheStruct()
    cs.struct_size = C.sizeof(cs)
    cs.B, cs.Hkv, cs.d, cs.n_sink, cs.n_recent, cs.mid_cap = 4096, 8, 128, 128, 256, 1 << 20
    need = L.fp4_attention_decode_workspace_size(32, C.byref(cs))
    assert need > 16 << 20
    fake = C.c_void_p(1 << 20)
    st = L.fp4_attention_decode_noalloc(fake, 32, C.byref(cs), 0.0, 2, fake, None, None)
    msg = L.fp4_last_error().decode()
    assert st == -2 and "scratch" in msg and str(need) in msg
    # invalid arguments are reported as by fp4_attention_decode
    assert L.fp4_attention_decode_noalloc(fake, 0, C.byref(cs), 0.0, 2, fake, None, None) == -1


def test_balance_options_are_validated(L):
    """The balance pair's options are refused before any launch when they do
    not fit (ScaleSearch page, Metodologia / ScaleSearchAttention)."""
    import block_scaled_fp4_amd as fp4
    fake = C.c_void_p(1 << 20)
    # quantizer: channel exponents need block_axis 0, exp_rows dividing rows, no AMAX mode, 0/1 negate
    ax1 = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 0, 1, 0, (C.c_uint32 * 4)(), fake, 0, 16)
    assert L.fp4_quantize(fake, 0, 32, 32, 32, C.byref(ax1), fake, fake, None, None, None, 0, None) == -1
    rows = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 0, 0, 0, (C.c_uint32 * 4)(), fake, 0, 3)
    assert L.fp4_quantize(fake, 0, 32, 32, 32, C.byref(rows), fake, fake, None, None, None, 0, None) == -1
    assert "exp_rows" in L.fp4_last_error().decode()
    amax = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 1, 0, 0, (C.c_uint32 * 4)(), fake, 0, 16)
    assert L.fp4_quantize(fake, 0, 32, 32, 32, C.byref(amax), fake, fake, None, fake, fake, 1 << 20, None) == -1
    neg = fp4.QuantOpts(C.sizeof(fp4.QuantOpts), 1, -2, 6, 0, 0, 0, (C.c_uint32 * 4)(), fake, 2, 16)
    assert L.fp4_quantize(fake, 0, 32, 32, 32, C.byref(neg), fake, fake, None, None, None, 0, None) == -1
    # attention: balance_qk needs the call's own quantization
    quant = dict(q_codes=fake, q_scales=fake, k_codes=fake, k_scales=fake, v_codes=fake, v_scales=fake)
    P = _prob(fp4, **quant)
    O = fp4._opts(True, 0.0, 128, True, -2, 6, 0, 128, fp4.FP32, balance=True)
    assert L.fp4_attention_fwd(C.byref(P), C.byref(O), fake, None, None, None, fake, 1 << 30, None) == -1
    assert "balance_qk" in L.fp4_last_error().decode()
    # the exponent entry point: shapes, dtype and workspace
    Pq = _prob(fp4)
    need = L.fp4_qk_balance_workspace_size(C.byref(Pq))
    assert need > 0
    assert L.fp4_qk_balance(C.byref(Pq), fake, fake, need - 1, None) == -3
    assert L.fp4_qk_balance(C.byref(Pq), None, fake, need, None) == -1
    P64 = _prob(fp4, d=96)
    assert L.fp4_qk_balance(C.byref(P64), fake, fake, 1 << 30, None) == -2


def test_strides_are_validated(L):
    """Strided q, k, v (fp4.h, fp4_attn_problem strides): token rows at least d
    apart, whole 16-byte rows, non-negative strides, one K/V head within 32-bit
    offsets; the MXFP4 entry point takes dense inputs only."""
    import block_scaled_fp4_amd as fp4
    fake = C.c_void_p(1 << 20)
    O = fp4._opts(True, 0.0, 128, True, -2, 6, 0, 128, fp4.FP32)

    def run(**st):
        P = _prob(fp4)
        for name, val in st.items():
            setattr(P, name, (C.c_int64 * 3)(*val))
        return L.fp4_attention_fwd(C.byref(P), C.byref(O), fake, None, None, None, fake, 1 << 40, None)

    d = 128
    assert run(q_strides=(0, d, d - 8)) == -1           # token stride below d
    assert "token stride" in L.fp4_last_error().decode()
    assert run(k_strides=(0, d, 3 * d + 4)) == -1       # rows not 16-byte aligned
    assert "multiples of 8" in L.fp4_last_error().decode()
    assert run(v_strides=(-8, d, 3 * d)) == -1          # negative stride
    assert run(k_strides=(0, 0, 1 << 30)) == -2         # one head past 32-bit offsets
    O_mx = fp4._opts(True, 0.0, 128, False, -2, 6, 0, 128, fp4.FP32)
    P = _prob(fp4)
    P.q_strides = (C.c_int64 * 3)(0, d, 3 * d)
    assert L.fp4_attention_fwd_mx(C.byref(P), C.byref(O_mx), fake, None, fake, 1 << 40, None) == -2
    assert "dense" in L.fp4_last_error().decode()


def test_binding_strides_of_views():
    """The binding passes a view's {batch, head, token} strides (zeros when
    dense; size-1 dimensions normalized) and refuses rows that are not
    contiguous."""
    import torch
    import block_scaled_fp4_amd as fp4
    B, S, H, Hkv, d = 2, 64, 4, 2, 128
    buf = torch.zeros((B, S, H + 2 * Hkv, d), dtype=torch.bfloat16)
    q = buf[:, :, :H].transpose(1, 2)
    assert list(fp4._strides(q)) == [S * (H + 2 * Hkv) * d, d, (H + 2 * Hkv) * d]
    assert list(fp4._strides(q.contiguous())) == [0, 0, 0]
    one = torch.zeros((1, 40, 1, d), dtype=torch.bfloat16)[:, ::2]  # B = 1, one token per head
    assert list(fp4._strides(one)) == [0, 2 * d, d]
    with pytest.raises(fp4.FP4Error, match="GPU"):
        fp4._dev_rows(q, "q")
