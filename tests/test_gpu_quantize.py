"""GPU quantizer parity: codes, scales, offsets and the per-tensor scale must be
bit-exact to the oracle (ScaleSearch page, Metodologia / ScaleSearch)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_amd import synth
from gpu_helpers import case

pytestmark = pytest.mark.gpu


def _run(fp4, x_cpu, axis, search, gmode=0, g=None, fmin=-2, fmax=6):
    x = x_cpu.cuda()
    gt = torch.tensor([g], dtype=torch.float32, device="cuda") if g is not None else None
    r = fp4.fp4_quantize(x, block_axis=axis, scale_search=search, f_min=fmin, f_max=fmax, global_scale=gmode, g=gt)
    torch.cuda.synchronize()
    o = oracle.quantize(x_cpu, axis, search, fmin, fmax, gmode, g if g is not None else 1.0)
    codes = r["codes"].cpu().numpy()
    scales = r["scales"].cpu().numpy()
    offs = r["offsets"].cpu().numpy()
    np.testing.assert_array_equal(scales, o["scales"])
    np.testing.assert_array_equal(offs, o["offsets"])
    np.testing.assert_array_equal(codes, o["codes"])
    if gmode != 0:
        assert r["g"].item() == np.float32(o["g"])
    return r


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("search", [False, True])
def test_small_shapes_bit_exact(gpu, dtype, axis, search):
    g = torch.Generator().manual_seed(11)
    rows, cols = (48, 80) if axis == 1 else (37, 96)
    x = (torch.randn(rows, cols, generator=g) * torch.logspace(-3, 3, cols)).to(dtype)
    case(f"quantize small {dtype} axis={axis} search={search}")
    _run(gpu, x, axis, search)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("cols", [18, 84, 4])
def test_rows_axis_column_groups(gpu, dtype, cols):
    # blocks along rows: four columns per lane when cols is a multiple of 4 (84, 4),
    # one column per lane otherwise (18); both bit-exact
    g = torch.Generator().manual_seed(13 + cols)
    x = (torch.randn(64, cols, generator=g) * torch.logspace(-2, 2, cols)).to(dtype)
    case(f"quantize axis=1 {dtype} cols={cols}")
    _run(gpu, x, 1, True)


@pytest.mark.parametrize("gmode", [1, 2])
def test_global_scale_modes(gpu, gmode):
    g = torch.Generator().manual_seed(12)
    x = (torch.randn(64, 128, generator=g) * 30).to(torch.bfloat16)
    case(f"quantize global mode {gmode}")
    _run(gpu, x, 0, True, gmode=gmode, g=0.0123 if gmode == 2 else None)
    _run(gpu, x, 1, True, gmode=gmode, g=0.0123 if gmode == 2 else None)


def test_special_values(gpu):
    x = torch.zeros(32, 64, dtype=torch.float32)
    x[0, :16] = -0.0
    x[1, 3] = float("inf")
    x[2, 20] = float("nan")
    x[3, :16] = torch.tensor([2.0 ** -140] * 16)          # scale underflows to 0
    x[4, :16] = 1e30                                       # saturates at 448
    x[5, :16] = torch.arange(16) * 0.25                    # exact grid midpoints
    x[6, :16] = 1.0                                        # worked example -> byte 0x28
    x[7, 16:32] = torch.tensor([6.0, -6.0] * 8) * 448      # top of the range
    case("quantize special values")
    r = _run(gpu, x, 0, True)
    assert r["scales"][6, 0].item() == 0x28
    _run(gpu, x, 0, False)
    _run(gpu, x.t().contiguous(), 1, True)


def test_scale_rounding_boundaries(gpu):
    """Blocks whose amax / 6 sits on or next to an E4M3 rounding point: ties
    between normal neighbours (even mantissa wins), ties in the subnormal
    range (steps of 2^-9), and the band between 448 and the next would-be
    step, where the scale byte saturates at 0x7E."""
    e4m3 = [k / 512 for k in range(8)] + [(1 + m / 8) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
    e4m3 = sorted(v for v in e4m3 if v <= 448)
    mids = [(a + b) / 2 for a, b in zip(e4m3, e4m3[1:])]
    picks = mids[:10] + mids[50:60] + mids[-10:] + [448.0, 452.0, 456.0, 460.0, 464.0, 466.0, 470.0, 480.0]
    amax = []
    for m in picks:  # the midpoint itself and its binary32 neighbours, times 6 (exact in binary32 or next to it)
        f = np.float32(m * 6)
        amax += [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(0))]
    x = torch.zeros(len(amax), 32, dtype=torch.float32)
    g = torch.Generator().manual_seed(21)
    for i, a in enumerate(amax):
        row = torch.rand(32, generator=g) * float(a)
        row[i % 16] = float(a)
        row[16 + (i * 7) % 16] = -float(a)
        x[i] = row
    case("quantize E4M3 rounding boundaries")
    _run(gpu, x, 0, True)
    _run(gpu, x, 0, False)


def test_offset_ranges(gpu):
    g = torch.Generator().manual_seed(13)
    x = torch.randn(64, 64, generator=g).to(torch.bfloat16)
    for fmin, fmax in ((-8, 8), (0, 0), (-1, 3), (0, 6)):
        case(f"quantize offset range [{fmin},{fmax}]")
        _run(gpu, x, 0, True, fmin=fmin, fmax=fmax)


def test_quantizer_workload_full_size(gpu):
    """bf16 [32768, 128] with 2% outlier channels x20, ScaleSearch, per-tensor amax scale."""
    x = synth.quant_tensor()
    case("quantize full workload 32768x128 bf16 amax scalesearch")
    r = _run(gpu, x, 0, True, gmode=1)
    # run twice: bitwise deterministic
    r2 = gpu.fp4_quantize(x.cuda(), 0, True, -2, 6, gpu.GLOBAL_AMAX)
    torch.cuda.synchronize()
    assert torch.equal(r["codes"], r2["codes"]) and torch.equal(r["scales"], r2["scales"])


def test_empty_input(gpu):
    x = torch.zeros(0, 32, dtype=torch.bfloat16, device="cuda")
    case("quantize empty")
    r = gpu.fp4_quantize(x, 0, True, -2, 6, gpu.GLOBAL_AMAX)
    torch.cuda.synchronize()
    assert r["codes"].numel() == 0 and r["g"].item() == 1.0
