"""Seeded random geometries against the fp64 oracle: every algorithm that
accepts a drawn convolution (forced, and AUTO), with random K splits, unfold
row caps and Winograd batch tiles, in all three dtypes, 2D and 3D.  The draws
are fixed by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import conv_workloads as cw
import oracle
from gpu_util import check_parity, poisoned, to_oracle

pytestmark = pytest.mark.gpu

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")

N_CASES = 256


def _extent(i, k, s, p, d):
    return (i + 2 * p - d * (k - 1) - 1) // s + 1


def draw_case(idx):
    """Case idx of the fixed sequence: a ConvCase plus the per-algorithm options."""
    g = np.random.default_rng([7, idx])
    nd = 3 if g.random() < 0.3 else 2
    dtype = ["f32", "f16", "bf16"][int(g.integers(3))]
    # about half the draws have the Winograd geometry (3x3, stride 1,
    # dilation 1, small padding, C >= 16), so those paths get their share
    wino = g.random() < 0.5
    while True:
        n = int(g.integers(1, 4))
        h, w = int(g.integers(1, 21)), int(g.integers(1, 21))
        k = 3 if wino else int(g.choice([1, 2, 3, 4, 5]))
        s = 1 if wino else int(g.choice([1, 1, 2, 3]))
        dl = 1 if wino else int(g.choice([1, 1, 2]))
        p = int(g.choice([0, 1, 1])) if wino else int(g.integers(0, 3))
        c = int(g.choice([16, 24, 32, 40, 64])) if wino else int(g.choice([int(g.integers(1, 70)), 16, 32, 64]))
        o = int(g.integers(1, 70))
        d, kd, sd, pd, dd = 1, 1, 1, 0, 1
        if nd == 3:
            d, kd = int(g.integers(1, 7)), int(g.integers(1, 4))
            sd = 1 if wino else int(g.choice([1, 1, 2]))
            pd, dd = int(g.integers(0, 2)), int(g.choice([1, 1, 2]))
            if wino and g.random() < 0.5:
                n, pd, dd = 1, 0, 1  # also the decomposition's structural guard
        if min(_extent(h, k, s, p, dl), _extent(w, k, s, p, dl), _extent(d, kd, sd, pd, dd)) >= 1:
            break
    if nd == 2:
        case = cw.ConvCase(f"fuzz{idx}", n, h, w, c, o, k, k, (s, s), (p, p), (dl, dl), dtype, "normal", "normal",
                           None, 77, idx)
    else:
        case = cw.ConvCase(f"fuzz{idx}", n, h, w, c, o, k, k, (sd, s, s), (pd, p, p), (dd, dl, dl), dtype, "normal",
                           "normal", None, 77, idx, nd=3, d=d, kd=kd)
    opts = {"split_k": int(g.integers(2, 5)), "unfold_rows": int(g.integers(1, 300)),
            "tile_batch": int(g.integers(1, 3))}
    return case, opts


def _runs(case, opts):
    """(label, kwargs) of every algorithm variant to try on this case."""
    runs = [("auto", {})]
    runs += [("implicit_gemm", dict(algo="implicit_gemm")),
             ("implicit_gemm_split", dict(algo="implicit_gemm", split_k=opts["split_k"]))]
    if case.nd == 2:
        runs += [("unfold_gemm", dict(algo="unfold_gemm")),
                 ("unfold_gemm_rows", dict(algo="unfold_gemm", unfold_rows=opts["unfold_rows"])),
                 ("winograd", dict(algo="winograd")),
                 ("winograd_tiled", dict(algo="winograd", tile_batch=opts["tile_batch"])),
                 ("winograd_half", dict(algo="winograd_half"))]
    else:
        runs += [("small_kd", dict(algo="small_kd")), ("winograd_half", dict(algo="winograd_half"))]
    return runs


@pytest.mark.parametrize("idx", range(N_CASES))
def test_fuzz_parity(idx):
    case, opts = draw_case(idx)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    fn = cn.conv2d if case.nd == 2 else cn.conv3d
    plan_fn = cn.plan2d if case.nd == 2 else cn.plan3d
    ran = 0
    for label, kw in _runs(case, opts):
        try:
            plan_fn(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, **kw)
        except cn.CnhwcError as e:
            assert e.name in ("NOT_APPLICABLE", "UNSUPPORTED"), (label, e.name)
            continue
        y = fn(x.cuda(), wt.cuda(), **case.conv_kwargs(), out=poisoned(yr.shape, x.dtype), **kw)
        check_parity(y.cpu(), yr, den, x.dtype, f"{case} / {label}")
        ran += 1
    assert ran >= 2
