"""GPU parity on inputs with zero regions: every output whose products x * w
are all zero (sum|x||w| == 0) must be exactly zero, on the Winograd paths as
well as the GEMM paths.  Elsewhere the GEMM paths and the fp32 F(6x6,3x3)
path meet the per-output bound; the half-precision F(4x4,3x3) path meets the
tile-relative bound (an output whose window holds one isolated pixel, in a
tile that reaches dense data, is 1/9 as bright as its neighbours, and with
few channels its fp16 rounding does not average down).

The Winograd transforms round every value of a tile at the scale of its
largest values, so an output whose window lies in a zero region of a tile
that also holds nonzero pixels would otherwise carry rounding residue.  The
inputs here are letterboxed (zero columns at the left), hold a zeroed block
with a few isolated nonzero pixels inside it, and (for batches of more than
one) a wholly zero image; the filters hold output channels whose only nonzero
tap is the centre (so outputs next to an isolated pixel see it only under zero
taps) and one all-zero output channel.  The algorithms and channel counts
cover both ways the input transform records its tile masks: whole wavefronts
per tile (Cs a multiple of 64 channel threads) and workgroups shared by
several tiles.
"""
import numpy as np
import pytest
import torch

import conv_workloads as cw
import oracle
from gpu_util import bits, check_parity, check_tile_relative, poisoned, to_oracle

pytestmark = pytest.mark.gpu

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")


def _zero_regions(x, nd):
    """Zero the left 12 columns, a block with isolated pixels left in it, and
    (batch >= 2) the whole last element; 3D: also two whole frames."""
    x = x.float().clone()
    w_axis = x.dim() - 2
    x.narrow(w_axis, 0, min(12, x.shape[w_axis])).zero_()
    sp = x[0] if nd == 2 else x[0, 1]
    h, w = sp.shape[0], sp.shape[1]
    r0, c0 = h // 3, max(14, w // 3)
    if c0 + 10 <= w and r0 + 10 <= h:
        keep = sp[r0 + 4, c0 + 5].clone(), sp[r0 + 7, c0 + 2].clone()
        sp[r0:r0 + 10, c0:c0 + 10] = 0
        sp[r0 + 4, c0 + 5], sp[r0 + 7, c0 + 2] = keep
    if x.shape[0] >= 2:
        x[-1] = 0
    if nd == 3 and x.shape[1] >= 6:
        x[:, 3:5] = 0
    return x


def _sparse_taps(wt):
    """Output channel 0: centre tap only; channel 1 (if any): all zero; the
    last channel: the top-left tap only."""
    wt = wt.float().clone()
    o = wt.shape[0]
    centre = wt[0].clone()
    wt[0] = 0
    if wt.dim() == 4:
        wt[0, 1, 1] = centre[1, 1]
        wt[-1, :, :] = torch.where(torch.arange(9).reshape(3, 3, 1) == 0, wt[-1], torch.zeros_like(wt[-1]))
    else:
        wt[0, :, 1, 1] = centre[:, 1, 1]
        wt[-1, :, :, :] = torch.where(torch.arange(9).reshape(1, 3, 3, 1) == 0, wt[-1], torch.zeros_like(wt[-1]))
    if o > 2:
        wt[1] = 0
    return wt


def _run(case, algo, **kw):
    x = _zero_regions(case.input(), case.nd).to(cw.DTYPES[case.dtype])
    wt = _sparse_taps(case.weight()).to(cw.DTYPES[case.dtype])
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    zero = den == 0
    assert zero.sum() > 0 and (~zero).sum() > 0, "the case must have zero and nonzero windows"
    fn = cn.conv2d if case.nd == 2 else cn.conv3d
    y = fn(x.cuda(), wt.cuda(), **case.conv_kwargs(), algo=algo, out=poisoned(yr.shape, x.dtype), **kw)
    torch.cuda.synchronize()
    inner = kw.get("inner_algo", algo)
    if algo == "winograd_half" or inner == "winograd_half":
        check_tile_relative(y.cpu(), yr, den, x.dtype, 4, f"{case.name}/{algo}")
    else:
        check_parity(y.cpu(), yr, den, x.dtype, f"{case.name}/{algo}")
    return x, wt, y


# (algo, dtype, n, h, w, c, o): mask mode in the comment (threads per tile row)
ZERO_2D = [
    ("winograd", "f32", 2, 30, 34, 64, 48),        # 64 threads per tile: wavefront parts
    ("winograd", "f32", 3, 26, 40, 192, 96),       # 192: three wavefront parts
    ("winograd", "f32", 2, 31, 29, 40, 24),        # 40: workgroup parts
    ("winograd", "f32", 1, 28, 30, 20, 16),        # Cs 24: workgroup parts, padded channels
    ("winograd", "bf16", 2, 27, 33, 32, 32),       # fp32 F(6x6,3x3) on bf16 data
    ("winograd_half", "f16", 2, 30, 34, 64, 48),   # 16 threads per tile: workgroup parts
    ("winograd_half", "bf16", 2, 26, 30, 256, 64),  # 64: one wavefront part
    ("winograd_half", "f16", 1, 33, 27, 512, 32),  # 128: two wavefront parts
    ("winograd_half", "bf16", 2, 25, 31, 30, 20),  # two channels per thread
    ("winograd_half", "f16", 2, 22, 26, 17, 16),   # one channel per thread
    ("implicit_gemm", "f32", 2, 30, 34, 64, 48),
    ("implicit_gemm", "bf16", 2, 30, 34, 64, 48),
    ("unfold_gemm", "f16", 2, 30, 34, 40, 24),
]


@pytest.mark.parametrize("spec", ZERO_2D, ids=[f"{s[0]}_{s[1]}_c{s[5]}" for s in ZERO_2D])
def test_zero_regions_exact_2d(spec):
    algo, dt, n, h, w, c, o = spec
    case = cw.ConvCase(f"zero2d_{algo}_{dt}_c{c}", n, h, w, c, o, 3, 3, (1, 1), (1, 1), (1, 1), dt,
                       "uniform" if dt == "f32" else "normal", "normal", None, 71, c + o)
    _run(case, algo)


def test_zero_regions_winograd_tiled_bit_identical():
    """Batch tiles keep the untiled bits with the masks in use."""
    case = cw.ConvCase("zero_tiles", 3, 30, 26, 64, 32, 3, 3, (1, 1), (1, 1), (1, 1), "f32", "uniform", "normal",
                       None, 72, 0)
    x, wt, y_full = _run(case, "winograd")
    for tile in (1, 2):
        y = cn.conv2d(x.cuda(), wt.cuda(), **case.conv_kwargs(), algo="winograd", tile_batch=tile)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_full)), f"tile {tile}"


def test_padding_only_windows_exact():
    """Padding 3 around a 3x3 filter: corner outputs see only padding, on a
    2x2 image whose tile holds the whole image."""
    for dt in ("f32", "bf16"):
        case = cw.ConvCase(f"pad3_{dt}", 2, 2, 2, 16, 7, 3, 3, (1, 1), (3, 3), (1, 1), dt, "normal", "normal",
                           None, 73, 0)
        x, wt = case.input(), case.weight()
        yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
        assert (den == 0).sum() > 0
        for algo in ("winograd", "implicit_gemm", "unfold_gemm", "auto"):
            y = cn.conv2d(x.cuda(), wt.cuda(), **case.conv_kwargs(), algo=algo, out=poisoned(yr.shape, x.dtype))
            torch.cuda.synchronize()
            check_parity(y.cpu(), yr, den, x.dtype, f"{case.name}/{algo}")


# (name, algo, inner, n, d, h, w, c, o, kd, pad, dil, dtype)
ZERO_3D = [
    ("wh_video", "winograd_half", "auto", 1, 7, 16, 22, 64, 64, 3, (0, 1, 1), (1, 1, 1), "bf16"),
    ("wh_pad_dil", "winograd_half", "auto", 2, 9, 14, 20, 64, 40, 3, (1, 1, 1), (2, 1, 1), "f16"),
    ("wh_wave", "winograd_half", "auto", 1, 6, 12, 26, 256, 32, 3, (1, 1, 1), (1, 1, 1), "bf16"),
    ("smallkd_wino", "small_kd", "winograd", 1, 7, 18, 26, 32, 32, 3, (0, 1, 1), (1, 1, 1), "f32"),
    ("smallkd_wino_bf16", "small_kd", "winograd", 1, 6, 14, 24, 64, 32, 2, (0, 1, 1), (1, 1, 1), "bf16"),
    ("native", "implicit_gemm", "auto", 1, 7, 16, 22, 64, 64, 3, (0, 1, 1), (1, 1, 1), "bf16"),
]


@pytest.mark.parametrize("spec", ZERO_3D, ids=[s[0] for s in ZERO_3D])
def test_zero_regions_exact_3d(spec):
    name, algo, inner, n, d, h, w, c, o, kd, pad, dil, dt = spec
    case = cw.ConvCase(f"zero3d_{name}", n, h, w, c, o, 3, 3, (1, 1, 1), pad, dil, dt,
                       "uniform" if dt == "f32" else "normal", "normal", None, 74, c + kd, nd=3, d=d, kd=kd)
    _run(case, algo, **({"inner_algo": inner} if inner != "auto" else {}))
