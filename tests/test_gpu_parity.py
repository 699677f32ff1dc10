"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Cases follow the workloads of the MLX pages: the small fp32 3x3 conv, the
half-precision filter/stride/dilation/padding grid with aligned and unaligned
channels (MLX PR "Use the explicit gemm for wide convs on neural accelerators",
Verified), the fp32 Winograd workload at reduced batch and size (MLX PR "Bound
winograd conv2d working set by tiling the batch"), and the 3D decomposition
(MLX PR "Decompose small kernel-depth 3D convs into 2D convs", Tests).
"""
import numpy as np
import pytest
import torch

import conv_workloads as cw
import oracle
from gpu_util import TOL, bits, check_parity, gather_rows, poisoned, tile_max, to_oracle

pytestmark = pytest.mark.gpu

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")


def _dev(t):
    return t.to("cuda")


def _run_case(case, algo, rows=None, **kw):
    w = case.weight()
    x = case.input()
    xg, wg = _dev(x), _dev(w)
    fn = cn.conv2d if case.nd == 2 else cn.conv3d
    y = fn(xg, wg, **case.conv_kwargs(), algo=algo, **kw)
    torch.cuda.synchronize()
    yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs(), rows=rows)
    yg = gather_rows(y, rows) if rows is not None else y.cpu()
    return check_parity(yg, yr, den, y.dtype, f"{case.name}/{algo}"), y


# ------------------------------------------------------------ small fp32 conv

@pytest.mark.parametrize("algo", ["winograd", "implicit_gemm", "unfold_gemm", "auto"])
def test_small_fp32_all_algorithms(algo):
    case = cw.small_fp32()
    err, y = _run_case(case, algo)
    assert err < 2e-5
    p = cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs())
    assert p.algo_name == "implicit_gemm"  # C+O = 64 < 256: AUTO does not take Winograd


# ------------------------------------------------------- half geometry grid

GRID = [(dt, c) for dt in ("f16", "bf16") for c in (128, 120)]


@pytest.mark.parametrize("dtype,c_in", GRID)
def test_half_geometry_grid(dtype, c_in):
    for case in cw.half_geometry_grid(dtype, c_in):
        x, w = case.input(), case.weight()
        yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs())
        for algo in ("implicit_gemm", "unfold_gemm"):
            y = cn.conv2d(_dev(x), _dev(w), **case.conv_kwargs(), algo=algo)
            check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/{algo}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c_in,k,s,p", [(3, 7, 2, 3), (5, 3, 1, 1), (3, 3, 2, 0)])
def test_half_small_channels(dtype, c_in, k, s, p):
    """Channel counts below one 16-byte vector (the 3-channel stem): the
    implicit GEMM and the unfold gather element by element."""
    h = 30
    case = cw.ConvCase(f"small_c{c_in}_k{k}s{s}p{p}_{dtype}", 2, h, h + 3, c_in, 40, k, k, (s, s), (p, p), (1, 1),
                       dtype, "normal", "normal", None, 12, c_in * 10 + k)
    x, w = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs())
    for algo in ("implicit_gemm", "unfold_gemm", "auto"):
        y = cn.conv2d(_dev(x), _dev(w), **case.conv_kwargs(), algo=algo)
        check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/{algo}")


@pytest.mark.parametrize("k,s,d,p", [(3, 1, 1, 1), (5, 2, 1, 2), (7, 2, 2, 0), (1, 2, 1, 0), (3, 2, 2, 2)])
def test_fp32_geometry(k, s, d, p):
    h = (16 - 1) * s + d * (k - 1) + 1 - 2 * p
    for c_in in (64, 30):
        case = cw.ConvCase(f"f32_k{k}s{s}d{d}p{p}_c{c_in}", 2, h, h + 1, c_in, 48, k, k, (s, s), (p, p), (d, d),
                           "f32", "uniform", "normal", None, 9, k * 100 + c_in)
        x, w = case.input(), case.weight()
        yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs())
        for algo in ("implicit_gemm", "unfold_gemm"):
            y = cn.conv2d(_dev(x), _dev(w), **case.conv_kwargs(), algo=algo)
            check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/{algo}")


# ------------------------------------------------------- degenerate geometries

# (name, n, h, w, c, o, k, stride, pad, dilation)
DEGENERATE = [
    ("pixel_1x1", 3, 1, 1, 1, 1, 1, 1, 0, 1),          # a scalar multiply per element
    ("one_channel_3x3", 2, 5, 7, 1, 1, 3, 1, 1, 1),
    ("kernel_is_image", 2, 5, 5, 8, 3, 5, 1, 0, 1),     # one output pixel
    ("stride_past_image", 1, 3, 4, 8, 5, 3, 5, 0, 1),   # OH = OW = 1
    ("padding_only_windows", 2, 2, 2, 16, 7, 3, 1, 3, 1),  # corner outputs see only padding
    ("padding_ring_1x1", 2, 3, 3, 16, 5, 1, 1, 2, 1),   # the outer two rings see only padding
    ("one_output_channel_wide_k", 1, 6, 6, 1000, 1, 3, 1, 1, 1),
    ("image_1x1_pad1", 2, 1, 1, 16, 20, 3, 1, 1, 1),    # one Winograd tile, 8 of 9 taps padding
    ("dilated_past_image", 1, 4, 4, 8, 4, 3, 1, 2, 3),  # taps land outside the image
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("spec", DEGENERATE, ids=[d[0] for d in DEGENERATE])
def test_degenerate_geometries(spec, dtype):
    """Tiny and extreme shapes on every algorithm that accepts them; outputs
    whose windows hold only padding must be exactly zero."""
    name, n, h, w, c, o, k, s, p, d = spec
    case = cw.ConvCase(f"deg_{name}_{dtype}", n, h, w, c, o, k, k, (s, s), (p, p), (d, d), dtype, "normal",
                       "normal", None, 17, c + o + k)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    algos = ["auto", "implicit_gemm", "unfold_gemm"]
    if k == 3 and s == 1 and d == 1:
        algos.append("winograd")
        if dtype != "f32" and p <= 1 and c >= 16:
            algos.append("winograd_half")
    for algo in algos:
        y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, out=poisoned(yr.shape, x.dtype))
        check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/{algo}")


def test_degenerate_conv1d_and_3d():
    """conv1d of length-1 signals; a 3D conv whose output has one frame."""
    x1 = torch.randn((3, 1, 24), dtype=torch.float16)
    w1 = torch.randn((5, 3, 24), dtype=torch.float16) / 8
    y1 = cn.conv1d(_dev(x1), _dev(w1), 1, 1)
    yr, den = oracle.conv(to_oracle(x1.unsqueeze(1)), to_oracle(w1.unsqueeze(1)), stride=(1, 1), padding=(0, 1),
                          dilation=(1, 1))
    check_parity(y1.unsqueeze(1).cpu(), yr, den, y1.dtype, "conv1d_len1")
    case = cw.ConvCase("deg3d", 1, 6, 5, 32, 16, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), "bf16", "normal", "normal",
                       None, 18, 0, nd=3, d=3, kd=3)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    for algo in ("auto", "implicit_gemm", "small_kd", "winograd_half"):
        y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, out=poisoned(yr.shape, x.dtype))
        assert y.shape[1] == 1
        check_parity(y.cpu(), yr, den, y.dtype, f"deg3d/{algo}")


# ------------------------------------------- integer data: exact in every dtype

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("algo", ["implicit_gemm", "unfold_gemm"])
def test_integer_data_bit_exact(dtype, algo):
    # entries in {-1,0,1}, K = 3*3*24 = 216 <= 256: every partial sum is an
    # integer of magnitude <= 216, exact in fp32/fp16/bf16 -> results must equal
    # the oracle exactly.  (Not the Winograd paths: their transforms have
    # fractional coefficients, so they are not exact by construction.)
    case = cw.ConvCase("ternary", 2, 13, 11, 24, 40, 3, 3, (1, 1), (1, 1), (1, 1), dtype, "ternary", "ternary",
                       1.0, 21, 0)
    x, w = case.input(), case.weight()
    y = cn.conv2d(_dev(x), _dev(w), **case.conv_kwargs(), algo=algo)
    yr, _ = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs())
    assert np.array_equal(y.cpu().double().numpy(), yr)


# --------------------------------------------------------- Winograd tiling

def _wino_case(n=5, h=40, w=44, c=64, o=96):
    return cw.ConvCase(f"wino_{n}x{h}x{w}_{c}to{o}", n, h, w, c, o, 3, 3, (1, 1), (1, 1), (1, 1),
                       "f32", "uniform", "normal", (1.0 / (9 * c)) ** 0.5, 2, 77)


def test_winograd_parity_fp32():
    case = _wino_case()
    err, _ = _run_case(case, "winograd")
    assert err < 2e-5


@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_winograd_tiled_bit_identical_to_untiled(tile):
    case = _wino_case()
    x, w = _dev(case.input()), _dev(case.weight())
    full = cn.conv2d(x, w, 1, 1, 1, algo="winograd")
    p = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, algo="winograd", tile_batch=tile)
    assert p.tile_batch == tile and p.n_tiles == -(-case.n // tile)
    tiled = cn.conv2d(x, w, 1, 1, 1, algo="winograd", tile_batch=tile, out=poisoned(full.shape, full.dtype))
    assert torch.equal(bits(tiled), bits(full))


def test_winograd_budget_injection_tiles_and_falls_back():
    # T = 16*17 = 272 tiles per image: a 2-element tile carries 544 GEMM rows,
    # above the MIN_TILE_ROWS floor, so the budget rule tiles instead of falling back
    case = _wino_case(n=6, h=96, w=100, c=128, o=128)
    x, w = _dev(case.input()), _dev(case.weight())
    full = cn.conv2d(x, w, 1, 1, 1)
    assert cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1).algo_name == "winograd"
    base = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, ws_limit=10**12)
    # a W leaving room for exactly two elements
    need = base.own_bytes + 2 * base.scratch_per_element
    wl = -(-need * 4 // 3) + 8
    p = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, ws_limit=wl)
    assert p.algo_name == "winograd" and p.tile_batch == 2 and p.n_tiles == 3
    tiled = cn.conv2d(x, w, 1, 1, 1, ws_limit=wl)
    assert torch.equal(bits(tiled), bits(full))
    # 1 MB -> implicit GEMM fallback: correct but not bit-identical in general
    p = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, ws_limit=2**20)
    assert p.algo_name == "implicit_gemm"
    fb = cn.conv2d(x, w, 1, 1, 1, ws_limit=2**20)
    yr, den = oracle.conv(to_oracle(case.input()), to_oracle(case.weight()), 1, 1, 1)
    check_parity(fb.cpu(), yr, den, torch.float32, "fallback")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_winograd_half_precision_forced(dtype):
    case = cw.ConvCase(f"wino_{dtype}", 2, 20, 23, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1), dtype, "normal",
                       "normal", None, 3, 5)
    err, _ = _run_case(case, "winograd")
    assert err < 1e-2


# ---------------------------------------------------------------- 3D

@pytest.mark.parametrize("kd", [1, 2, 3, 5])
@pytest.mark.parametrize("inner", ["auto", "implicit_gemm", "winograd", "unfold_gemm"])
def test_conv3d_small_kd(kd, inner):
    case = cw.ConvCase(f"c3d_kd{kd}", 1, 9, 10, 32, 48, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), "bf16",
                       "normal", "normal", None, 5, kd, nd=3, d=kd + 4, kd=kd)
    err, _ = _run_case(case, "small_kd", inner_algo=inner)
    assert err < 1e-2


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_conv3d_kd1_bit_identical_to_conv2d(dtype):
    case = cw.ConvCase("c3d_kd1", 1, 12, 12, 32, 32, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), dtype,
                       "normal", "normal", None, 5, 99, nd=3, d=6, kd=1)
    x, w = _dev(case.input()), _dev(case.weight())
    y3 = cn.conv3d(x, w, 1, (0, 1, 1), 1)
    y2 = cn.conv2d(x[0], w[:, 0].contiguous(), 1, 1, 1)
    assert torch.equal(bits(y3[0]), bits(y2))


# ------------------------------- 256x256 tile with direct loads into LDS
# Shapes chosen to span several row and column tiles with ragged tails, every
# filter geometry of the half grid, and C = 32 / 64 / 96 / 128 (the tile needs
# C % 32 == 0 for the implicit gather, K % 8 == 0 for unfold rows; with
# C % 64 == 0 the 256 x 256 tile gathers in 64-element chunks, so both of its
# chunk forms are compared with the 128 x 128 tile's bits).

LDS_CASES = [  # name, n, h, w, c, o, k, stride, pad, dil
    ("c64_o300", 2, 20, 20, 64, 300, 3, 1, 1, 1),
    ("c96_s2", 3, 33, 31, 96, 260, 3, 2, 1, 1),
    ("c32_k5_d2", 2, 24, 24, 32, 256, 5, 1, 4, 2),
    ("c128_k1", 1, 30, 30, 128, 520, 1, 1, 0, 1),
    ("c64_k7_s2", 2, 40, 40, 64, 64, 7, 2, 3, 1),
    ("c32_k1_one_chunk", 1, 17, 15, 32, 96, 1, 1, 0, 1),
]


@pytest.mark.parametrize("tile", [14, 15])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("spec", LDS_CASES, ids=[c[0] for c in LDS_CASES])
def test_lds_tile_parity(dtype, spec, tile):
    name, n, h, w, c, o, k, s, p, d = spec
    case = cw.ConvCase(f"lds_{name}_{dtype}", n, h, w, c, o, k, k, (s, s), (p, p), (d, d), dtype,
                       "normal", "normal", None, 21, len(name) * 7 + c)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    for algo in ("implicit_gemm", "unfold_gemm"):
        plan = cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo=algo,
                         gemm_config=tile)
        assert plan.kernel_config == tile
        y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, gemm_config=tile)
        check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/{algo}/cfg{tile}")
        # same K order as the 128x128 tile (unsplit): bit-identical results
        y11 = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, gemm_config=11, split_k=1)
        assert torch.equal(bits(y), bits(y11)), f"{case.name}/{algo}: cfg {tile} and 128x128 tiles differ"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_lds_tile_3d_accumulating_epilogue(dtype):
    """Per-tap 2D convs of the 3D decomposition accumulate in fp32 through the
    256x256 tile's epilogue modes (first / middle / last tap)."""
    case = cw.ConvCase(f"lds3d_{dtype}", 1, 18, 19, 64, 272, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), dtype,
                       "normal", "normal", None, 23, 5, nd=3, d=6, kd=3)
    x, wt = case.input(), case.weight()
    plan = cn.plan3d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="small_kd",
                     gemm_config=14)
    assert plan.algo_name == "small_kd" and plan.kernel_config == 14
    y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="small_kd", gemm_config=14)
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    check_parity(y.cpu(), yr, den, y.dtype, case.name)
    y11 = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="small_kd", gemm_config=11, split_k=1)
    assert torch.equal(bits(y), bits(y11))


# ------------------------------- implicit GEMM from input patches staged in LDS
# Config 16: 3x3 stride-1 convs with C % 64 == 0; each 256-pixel block's input
# patch is loaded once per 64 channels and all nine taps read it.  Shapes span
# several blocks and column tiles with ragged tails, all three block widths
# (16 x 16, 8 x 32 for wide images, 32 x 8 for narrow ones), padding 0 and 1,
# images smaller than one block, and 3D with depth padding, stride and dilation.

PATCH_CASES = [  # name, n, h, w, c, o, pad
    ("c64_o300", 2, 20, 20, 64, 300, 1),
    ("c128_o256_p0", 1, 33, 35, 128, 256, 0),
    ("c192_o520_ragged", 3, 17, 29, 192, 520, 1),
    ("c64_tiny", 2, 5, 3, 64, 70, 1),
    ("c64_wide", 1, 6, 70, 64, 256, 1),
    ("c256_narrow", 1, 70, 5, 256, 96, 1),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("spec", PATCH_CASES, ids=[c[0] for c in PATCH_CASES])
def test_patch_tile_parity(dtype, spec):
    name, n, h, w, c, o, p = spec
    case = cw.ConvCase(f"patch_{name}_{dtype}", n, h, w, c, o, 3, 3, (1, 1), (p, p), (1, 1), dtype,
                       "normal", "normal", None, 29, len(name) * 3 + c)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    plan = cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="implicit_gemm",
                     gemm_config=16)
    assert plan.kernel_config == 16
    y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), plan=plan, out=poisoned(yr.shape, x.dtype))
    check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/cfg16")
    y2 = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), plan=plan)
    assert torch.equal(bits(y), bits(y2)), f"{case.name}: run-to-run bits differ"


PATCH3D_CASES = [  # name, n, d, h, w, c, o, kd, stride, pad, dil, dtype
    ("video_like", 1, 7, 20, 22, 64, 288, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), "bf16"),
    ("pad_d_batch2", 2, 6, 9, 10, 64, 80, 3, (1, 1, 1), (1, 1, 1), (1, 1, 1), "f16"),
    ("stride_d2_dil_d2", 1, 11, 12, 19, 128, 64, 3, (2, 1, 1), (1, 0, 1), (2, 1, 1), "bf16"),
    ("kd1", 2, 3, 17, 9, 64, 256, 1, (1, 1, 1), (0, 1, 1), (1, 1, 1), "f16"),
]


@pytest.mark.parametrize("spec", PATCH3D_CASES, ids=[c[0] for c in PATCH3D_CASES])
def test_patch_tile_3d_parity(spec):
    name, n, d, h, w, c, o, kd, s_, p_, dl, dt = spec
    case = cw.ConvCase(f"patch3d_{name}", n, h, w, c, o, 3, 3, s_, p_, dl, dt, "normal", "normal", None, 31,
                       len(name) + c, nd=3, d=d, kd=kd)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    plan = cn.plan3d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="implicit_gemm",
                     gemm_config=16)
    assert plan.kernel_config == 16
    y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), plan=plan, out=poisoned(yr.shape, x.dtype))
    check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/cfg16")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_patch_tile_accumulating_epilogue(dtype):
    """The per-tap 2D convs of the 3D decomposition through config 16 (first /
    middle / last tap epilogues), and KD = 1 giving conv2d's bits."""
    case = cw.ConvCase(f"patchkd_{dtype}", 1, 18, 19, 64, 272, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), dtype,
                       "normal", "normal", None, 33, 5, nd=3, d=6, kd=3)
    x, wt = case.input(), case.weight()
    plan = cn.plan3d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="small_kd",
                     inner_algo="implicit_gemm", gemm_config=16)
    assert plan.algo_name == "small_kd" and plan.kernel_config == 16
    y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), plan=plan)
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    check_parity(y.cpu(), yr, den, y.dtype, case.name)
    x1, w1 = _dev(x[:, :4]), _dev(wt[:, :1].contiguous())
    y3 = cn.conv3d(x1, w1, 1, (0, 1, 1), 1, algo="implicit_gemm", gemm_config=16)
    y2 = cn.conv2d(x1[0], w1[:, 0].contiguous(), 1, 1, 1, algo="implicit_gemm", gemm_config=16)
    assert torch.equal(bits(y3[0]), bits(y2))


# More tiles than compute units: each persistent workgroup of config 16 runs
# several tiles, loading the next tile's patch and first weight stages during
# its current tile's last (depth tap, chunk) iteration.  One iteration per
# tile (C = 64, KD = 1), odd iteration counts, two column tiles, ragged
# blocks, whole tiles only, 3D depth taps and the accumulating epilogues; a
# seeded sample of output pixels (with every pixel of the first and last
# blocks) against the oracle, every output written (the buffer starts as NaN)
# and the same bits on every run.
PERSIST_CASES = [  # name, n, d, h, w, c, o, kd, pad, dtype, algo
    ("c64_nit1", 70, 1, 32, 32, 64, 96, 0, (1, 1), "f16", "implicit_gemm"),
    ("c64_o512_whole_tiles", 40, 1, 32, 32, 64, 512, 0, (1, 1), "f16", "implicit_gemm"),
    ("c128_o256_whole_tiles", 72, 1, 32, 32, 128, 256, 0, (1, 1), "bf16", "implicit_gemm"),
    ("c192_o300_ragged", 24, 1, 33, 35, 192, 300, 0, (1, 1), "bf16", "implicit_gemm"),
    ("video_kd3", 1, 20, 64, 64, 128, 64, 3, (0, 1, 1), "bf16", "implicit_gemm"),
    ("small_kd_acc", 1, 19, 64, 64, 64, 72, 3, (0, 1, 1), "f16", "small_kd"),
]


@pytest.mark.parametrize("spec", PERSIST_CASES, ids=[c[0] for c in PERSIST_CASES])
def test_patch_tile_persistent(spec):
    name, n, d, h, w, c, o, kd, pad, dt, algo = spec
    nd = 3 if kd else 2
    stride, dil = (1,) * nd, (1,) * nd
    case = cw.ConvCase(f"persist_{name}", n, h, w, c, o, 3, 3, stride, pad, dil, dt, "normal", "normal", None, 37,
                       len(name) + c, nd=nd, d=d if kd else 1, kd=kd or 1)
    x, wt = case.input(), case.weight()
    kw = dict(algo=algo, gemm_config=16)
    if algo == "small_kd":
        kw["inner_algo"] = "implicit_gemm"
    plan = (cn.plan3d if nd == 3 else cn.plan2d)(case.x_shape(), case.w_shape(), **case.conv_kwargs(),
                                                 dtype=x.dtype, **kw)
    assert plan.kernel_config == 16
    per = plan.out_h * plan.out_w
    frames = n * (plan.out_d if nd == 3 else 1)
    assert _patch_tiles(frames, plan.out_h, plan.out_w) * -(-o // 256) > 256, "more tiles than CUs"
    fn = cn.conv3d if nd == 3 else cn.conv2d
    y = fn(_dev(x), _dev(wt), **case.conv_kwargs(), plan=plan, out=poisoned(plan_out_shape(plan, case), x.dtype))
    torch.cuda.synchronize()
    assert not torch.isnan(y).any(), "every output is written"
    total = frames * per
    rows = set(cw.sample_rows(total, 1500, 37).tolist())
    rows.update(range(0, 2 * plan.out_w))
    rows.update(range(total - 2 * plan.out_w, total))
    rows = np.array(sorted(rows), dtype=np.int64)
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs(), rows=rows)
    check_parity(gather_rows(y, rows), yr, den, x.dtype, case.name)
    y2 = fn(_dev(x), _dev(wt), **case.conv_kwargs(), plan=plan)
    assert torch.equal(bits(y), bits(y2)), f"{case.name}: run-to-run bits differ"


def _patch_tiles(frames, oh, ow):
    """Row tiles of config 16: blocks of the least padded width among 16, 32, 8."""
    best = None
    for bw in (16, 32, 8):
        bh = 256 // bw
        area = -(-oh // bh) * bh * -(-ow // bw) * bw
        if best is None or area < best[0]:
            best = (area, bw, bh)
    _, bw, bh = best
    return frames * -(-oh // bh) * -(-ow // bw)


def plan_out_shape(plan, case):
    if case.nd == 3:
        return (case.n, plan.out_d, plan.out_h, plan.out_w, case.o)
    return (case.n, plan.out_h, plan.out_w, case.o)


# ---------------------------------------------------------------- split K
# Small-grid GEMMs split K; the partial sums are added in a fixed order by a
# second kernel.  Forced splits (including a short last split) on every dtype
# and path, against the oracle, and the same bits on every run.

SPLIT_CASES = [  # name, n, h, w, c, o, k, stride, pad, dil, dtype
    ("l4_7x7_512", 1, 7, 7, 512, 512, 3, 1, 1, 1, "f16"),
    ("c120_unaligned", 1, 9, 11, 120, 72, 3, 1, 1, 1, "bf16"),
    ("s2_d2", 1, 21, 19, 64, 96, 5, 2, 2, 2, "bf16"),
    ("f32_small", 1, 16, 16, 32, 32, 3, 1, 1, 1, "f32"),
    ("f32_c30", 2, 10, 9, 30, 40, 3, 1, 1, 1, "f32"),
]


@pytest.mark.parametrize("spec", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_k_parity(spec):
    name, n, h, w, c, o, k, s, p, d, dt = spec
    case = cw.ConvCase(f"split_{name}", n, h, w, c, o, k, k, (s, s), (p, p), (d, d), dt,
                       "normal", "normal", None, 31, len(name) + c)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    for algo in ("implicit_gemm", "unfold_gemm"):
        for sk in (2, 3, 5):
            plan = cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo=algo,
                             split_k=sk)
            if plan.split_k < 2:
                continue
            y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, split_k=sk)
            check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/{algo}/split{plan.split_k}")
            y2 = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, split_k=sk)
            assert torch.equal(bits(y), bits(y2)), f"{case.name}/{algo}/split{sk}: run-to-run bits differ"


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_split_k_3d_accumulating_epilogue(dtype):
    """Per-tap 2D convs of the 3D decomposition through split GEMMs: the sum
    kernel applies the first / middle / last tap epilogues."""
    case = cw.ConvCase(f"split3d_{dtype}", 1, 6, 7, 64, 48, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), dtype,
                       "normal", "normal", None, 37, 3, nd=3, d=5, kd=3)
    x, wt = case.input(), case.weight()
    plan = cn.plan3d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="small_kd",
                     split_k=3)
    assert plan.algo_name == "small_kd" and plan.split_k == 3
    y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="small_kd", split_k=3)
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    check_parity(y.cpu(), yr, den, y.dtype, case.name)


# ------------------------------------------------- native 3D implicit GEMM
# One GEMM with K = KD*KH*KW*C over the NDHWC gather: the fall-through for 3D
# convs the decomposition does not take (batch > 1, depth stride, padding,
# dilation) and the decomposition with its taps fused.

NATIVE3D_CASES = [  # name, n, d, h, w, c, o, (kd, kh, kw), stride, pad, dil, dtype, gemm_config
    ("n2_pad_d", 2, 6, 9, 10, 64, 80, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "bf16", 0),
    ("stride_d2", 1, 9, 12, 11, 32, 48, (3, 3, 3), (2, 1, 2), (0, 1, 1), (1, 1, 1), "f16", 0),
    ("dil2_k5d", 1, 12, 8, 8, 64, 64, (5, 3, 3), (1, 1, 1), (2, 1, 1), (2, 1, 2), "bf16", 0),
    ("c40_scalar", 2, 5, 7, 9, 40, 24, (2, 3, 3), (1, 2, 1), (1, 0, 1), (1, 1, 1), "f16", 0),
    ("f32", 2, 5, 8, 7, 32, 40, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "f32", 0),
    ("f32_c6", 1, 6, 7, 8, 6, 10, (3, 2, 3), (1, 1, 1), (0, 1, 0), (1, 1, 1), "f32", 0),
    ("lds_tile", 1, 7, 20, 22, 64, 288, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "bf16", 14),
    ("lds_tile_s2", 2, 8, 17, 15, 32, 256, (3, 3, 3), (2, 2, 1), (1, 1, 1), (1, 1, 2), "f16", 14),
    ("lds_tile128", 1, 6, 19, 21, 96, 200, (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "bf16", 15),
    ("cfg11_split", 1, 5, 9, 9, 64, 96, (3, 3, 3), (1, 1, 1), (0, 1, 1), (1, 1, 1), "f16", 11),
]


@pytest.mark.parametrize("spec", NATIVE3D_CASES, ids=[c[0] for c in NATIVE3D_CASES])
def test_native3d_parity(spec):
    name, n, d, h, w, c, o, (kd, kh, kw), s, p, dl, dt, cfg = spec
    case = cw.ConvCase(f"native3d_{name}", n, h, w, c, o, kh, kw, s, p, dl, dt, "normal", "normal", None,
                       41, len(name) + c, nd=3, d=d, kd=kd)
    x, wt = case.input(), case.weight()
    kw_ = dict(gemm_config=cfg or None)
    splits = (None, 1, 3) if name == "cfg11_split" else (None, 1)
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    for sk in splits:
        plan = cn.plan3d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype,
                         algo="implicit_gemm", split_k=sk, **kw_)
        assert plan.algo_name == "implicit_gemm"
        if cfg:
            assert plan.kernel_config == cfg
        y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="implicit_gemm", split_k=sk, **kw_)
        check_parity(y.cpu(), yr, den, y.dtype, f"{case.name}/split{plan.split_k}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_native3d_depth1_bit_identical_to_conv2d(dtype):
    """D = KD = 1: the native 3D GEMM is the 2D implicit GEMM row for row."""
    case = cw.ConvCase(f"native3d_d1_{dtype}", 2, 10, 11, 64, 48, 3, 3, (1, 1), (1, 1), (1, 1), dtype,
                       "normal", "normal", None, 43, 1)
    x, wt = _dev(case.input()), _dev(case.weight())
    y2 = cn.conv2d(x, wt, 1, 1, 1, algo="implicit_gemm")
    y3 = cn.conv3d(x.unsqueeze(1), wt.unsqueeze(1), 1, (0, 1, 1), 1, algo="implicit_gemm")
    assert torch.equal(bits(y3.squeeze(1)), bits(y2))


# ------------------------------------------------------------------ conv1d
# conv1d routed through the 2D path (H = KH = 1): Whisper-encoder-shaped convs
# (log-mel -> d_model, k3 p1; d_model -> d_model, k3 s2 p1, 3000 frames) and
# odd geometries.

CONV1D_CASES = [  # name, n, l, c, o, k, stride, pad, dil, dtype
    ("enc_conv1", 1, 3000, 80, 384, 3, 1, 1, 1, "f16"),
    ("enc_conv2", 1, 3000, 384, 384, 3, 2, 1, 1, "f16"),
    ("enc_conv2_bf16_b2", 2, 1000, 512, 512, 3, 2, 1, 1, "bf16"),
    ("f32_k5_d2", 3, 77, 24, 40, 5, 1, 4, 2, "f32"),
    ("c7_k1", 2, 50, 7, 9, 1, 1, 0, 1, "f16"),
]


@pytest.mark.parametrize("spec", CONV1D_CASES, ids=[c[0] for c in CONV1D_CASES])
def test_conv1d_parity(spec):
    name, n, l, c, o, k, s, p, d, dt = spec
    case = cw.ConvCase(f"conv1d_{name}", n, 1, l, c, o, 1, k, (1, s), (0, p), (1, d), dt,
                       "normal", "normal", None, 51, len(name) + c)
    x, wt = case.input(), case.weight()                      # [N,1,L,C], [O,1,K,C]
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    y = cn.conv1d(_dev(x[:, 0]), _dev(wt[:, 0]), s, p, d)   # [N,OL,O]
    assert y.shape == (n, yr.shape[2], o)
    check_parity(y.cpu().unsqueeze(1), yr, den, y.dtype, case.name)


# -------------------------------------------------------------- HIP graphs
# The forward calls only queue kernels on the caller's stream (no allocation,
# no synchronisation, no memset), so a caller can capture them into a graph.
# Each replay must give the eager bits; eager work runs between replays.

def test_graph_capture_replays_bit_identical():
    cases = [  # (fn, case, kwargs): split-K implicit GEMM, native 3D, Winograd, half Winograd 2D/3D,
        # and the persistent patch-staged GEMM with more tiles than CUs
        (cn.conv2d, cw.ConvCase("g_l4", 1, 7, 7, 512, 512, 3, 3, (1, 1), (1, 1), (1, 1), "f16",
                                "normal", "normal", None, 61, 1), {}),
        (cn.conv2d, cw.ConvCase("g_patch", 70, 32, 32, 64, 96, 3, 3, (1, 1), (1, 1), (1, 1), "f16",
                                "normal", "normal", None, 66, 6), {"algo": "implicit_gemm", "gemm_config": 16}),
        (cn.conv3d, cw.ConvCase("g_3d", 2, 8, 9, 64, 48, 3, 3, (1, 1, 1), (1, 1, 1), (1, 1, 1), "bf16",
                                "normal", "normal", None, 62, 2, nd=3, d=5, kd=3), {}),
        (cn.conv2d, cw.ConvCase("g_wino", 2, 30, 30, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1), "f32",
                                "uniform", "normal", None, 63, 3), {"algo": "winograd"}),
        (cn.conv2d, cw.ConvCase("g_wino_half", 2, 30, 30, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1), "f16",
                                "normal", "normal", None, 64, 4), {"algo": "winograd_half"}),
        (cn.conv3d, cw.ConvCase("g_wino_half_3d", 1, 12, 14, 64, 48, 3, 3, (1, 1, 1), (1, 1, 1), (1, 1, 1),
                                "bf16", "normal", "normal", None, 65, 5, nd=3, d=6, kd=3),
         {"algo": "winograd_half"}),
    ]
    runs = []
    for fn, case, kw in cases:
        x, w = _dev(case.input()), _dev(case.weight())
        mk = cn.plan2d if case.nd == 2 else cn.plan3d
        plan = mk(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(), dtype=x.dtype, **kw)
        ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device="cuda")
        eager = fn(x, w, **case.conv_kwargs(), plan=plan, workspace=ws)
        out = torch.empty_like(eager)
        runs.append((fn, case, x, w, plan, ws, eager, out))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for fn, case, x, w, plan, ws, eager, out in runs:  # warm up on the capture stream
            fn(x, w, **case.conv_kwargs(), plan=plan, workspace=ws, out=out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for fn, case, x, w, plan, ws, eager, out in runs:
                fn(x, w, **case.conv_kwargs(), plan=plan, workspace=ws, out=out)
    for rep in range(3):
        for *_, out in runs:
            out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for fn, case, x, w, plan, ws, eager, out in runs:
            assert torch.equal(bits(out), bits(eager)), f"replay {rep}: {case.name} differs from eager"
        # eager work between replays, on the same buffers
        fn, case, x, w, plan, ws, eager, out = runs[0]
        fn(x, w, **case.conv_kwargs(), plan=plan, workspace=ws, out=out)
        torch.cuda.synchronize()


# ------------------------------- half-precision Winograd F(4x4,3x3)

# (name, n, h, w, c, o, pad, dtype, gemm tile): ragged 4x4 output tiles, odd
# channel counts (one channel per thread, padded K), C = 2 mod 4 (two per
# thread), padding 0, the fewest channels the path takes (16), and a case
# spanning several 256-row GEMM tiles with ragged rows and columns.
WH2D_CASES = [
    ("ragged_f16", 3, 21, 19, 64, 96, 1, "f16", 0),
    ("ragged_bf16", 3, 21, 19, 64, 96, 1, "bf16", 0),
    ("odd_channels_f16", 2, 13, 15, 37, 45, 1, "f16", 0),
    ("odd_channels_bf16", 2, 13, 15, 37, 45, 1, "bf16", 0),
    ("pad0_bf16", 2, 18, 18, 128, 64, 0, "bf16", 0),
    ("c16_f16", 2, 30, 30, 16, 32, 1, "f16", 0),
    ("c50_bf16", 2, 17, 19, 50, 40, 1, "bf16", 0),
    ("tiles_f16", 4, 64, 60, 256, 320, 1, "f16", 14),
    ("tiles_bf16", 4, 64, 60, 256, 320, 1, "bf16", 15),
]
# fp16 storage of the transformed operands costs about 2e-3 of sum|x||w|; the
# bf16 output rounding adds up to 2e-3 more.
WH_BOUND = {torch.float16: 5e-3, torch.bfloat16: 8e-3}


@pytest.mark.parametrize("spec", WH2D_CASES, ids=[c[0] for c in WH2D_CASES])
def test_winograd_half_parity(spec):
    name, n, h, w, c, o, pad, dt, cfg = spec
    case = cw.ConvCase(f"wh_{name}", n, h, w, c, o, 3, 3, (1, 1), (pad, pad), (1, 1), dt, "normal", "normal",
                       None, 61, c + o)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    plan = cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="winograd_half",
                     gemm_config=cfg or None)
    assert plan.algo_name == "winograd_half"
    y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="winograd_half", gemm_config=cfg or None,
                  out=poisoned(yr.shape, x.dtype))
    err = check_parity(y.cpu(), yr, den, y.dtype, case.name)
    assert err < WH_BOUND[y.dtype], err
    if cfg:
        # the two 256-row tiles sum K in the same order: identical bits
        other = 29 - cfg
        y2 = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="winograd_half", gemm_config=other)
        assert torch.equal(bits(y2), bits(y))


@pytest.mark.parametrize("tile", [1, 2, 3])
def test_winograd_half_tiled_bit_identical_to_untiled(tile):
    """The scales come from the whole tensors, so batch tiles keep the untiled bits."""
    case = cw.ConvCase("wh_tiling", 5, 24, 28, 64, 96, 3, 3, (1, 1), (1, 1), (1, 1), "f16", "normal", "normal",
                       None, 62, 0)
    x, w = _dev(case.input()), _dev(case.weight())
    full = cn.conv2d(x, w, 1, 1, 1, algo="winograd_half")
    p = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, torch.float16, algo="winograd_half", tile_batch=tile)
    assert p.tile_batch == tile and p.n_tiles == -(-case.n // tile)
    tiled = cn.conv2d(x, w, 1, 1, 1, algo="winograd_half", tile_batch=tile, out=poisoned(full.shape, full.dtype))
    assert torch.equal(bits(tiled), bits(full))


@pytest.mark.parametrize("dt,scale", [("f16", 6.0e4), ("f16", 1.0e-3), ("bf16", 1.0e30), ("bf16", 1.0e37),
                                      ("bf16", 1.0e-30), ("f16", 0.0)])
def test_winograd_half_input_range(dt, scale):
    """Inputs near the top of fp16's range (|B^T d B| would reach 6e6 unscaled),
    far outside it (bf16; at 1e37 even the fp32 transform of unscaled inputs
    would overflow), tiny, and all zero: the power-of-two scales keep every
    transformed value finite and the result within tolerance.  The weights are
    small enough (std 0.1/sqrt(K)) that y itself stays in fp16."""
    case = cw.ConvCase(f"wh_range_{dt}", 2, 14, 13, 64, 40, 3, 3, (1, 1), (1, 1), (1, 1), dt, "uniform", "normal",
                       0.1 / (9 * 64) ** 0.5, 63, 0)
    x = (case.input().float() * scale).to(cw.DTYPES[dt])
    wt = case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="winograd_half")
    err = check_parity(y.cpu(), yr, den, y.dtype, case.name + f"x{scale}")
    assert err < WH_BOUND[y.dtype], err


@pytest.mark.parametrize("algo,dt,tile", [("winograd", "f32", 6), ("winograd_half", "f16", 4),
                                          ("winograd_half", "bf16", 4), ("implicit_gemm", "f32", 1),
                                          ("implicit_gemm", "bf16", 1)])
@pytest.mark.parametrize("contrast", [0.1, 1e-3])
def test_winograd_error_is_tile_relative(algo, dt, tile, contrast):
    """A sharp edge: the left 11 columns of every image are `contrast` times
    smaller than the rest.  The Winograd transforms round each tile's values
    at the scale of the largest ones in it, so an output whose own window is
    dim but whose tile reaches the bright side carries an error relative to
    the tile: |err| <= tol * (largest sum|x||w| among its tile's outputs).
    At 10x contrast that is still within the per-output bound; the implicit
    GEMM meets the per-output bound at any contrast."""
    case = cw.ConvCase(f"edge_{algo}_{dt}", 2, 26, 27, 32, 24, 3, 3, (1, 1), (1, 1), (1, 1), dt, "uniform",
                       "normal", None, 91, 0)
    x = case.input().float()
    x[:, :, :11] *= contrast
    x = x.to(cw.DTYPES[dt])
    wt = case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    y = cn.conv2d(_dev(x), _dev(wt), **case.conv_kwargs(), algo=algo, out=poisoned(yr.shape, x.dtype))
    err = np.abs(y.cpu().double().numpy() - yr)
    tol = TOL[x.dtype]
    assert np.all(err <= tol * tile_max(den, tile)), float((err / tile_max(den, tile)).max())
    if contrast >= 0.1 or algo == "implicit_gemm":
        check_parity(y.cpu(), yr, den, x.dtype, case.name)


# (name, n, d, h, w, c, o, kd, pad (d, h, w), dilation (d, h, w), dtype)
WH3D_CASES = [
    ("video_like", 1, 7, 16, 20, 64, 64, 3, (0, 1, 1), (1, 1, 1), "bf16"),
    ("pad_d", 1, 6, 11, 13, 32, 48, 3, (1, 1, 1), (1, 1, 1), "f16"),
    ("dil_d2_batch2", 2, 9, 10, 12, 64, 40, 3, (1, 0, 1), (2, 1, 1), "bf16"),
    ("kd5_odd_o", 2, 8, 9, 9, 40, 33, 5, (2, 1, 1), (1, 1, 1), "f16"),
    ("kd1", 1, 5, 12, 14, 64, 64, 1, (0, 1, 1), (1, 1, 1), "bf16"),
]


@pytest.mark.parametrize("spec", WH3D_CASES, ids=[c[0] for c in WH3D_CASES])
def test_winograd_half_3d_parity(spec):
    """The depth taps summed inside the tile-position GEMMs (K = KD * Cs, tap kd
    reading the transformed frames kd * dilation further on)."""
    name, n, d, h, w, c, o, kd, pad, dil, dt = spec
    case = cw.ConvCase(f"wh3d_{name}", n, h, w, c, o, 3, 3, (1, 1, 1), pad, dil, dt, "normal", "normal", None,
                       64, c + kd, nd=3, d=d, kd=kd)
    x, wt = case.input(), case.weight()
    yr, den = oracle.conv(to_oracle(x), to_oracle(wt), **case.conv_kwargs())
    plan = cn.plan3d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=x.dtype, algo="winograd_half")
    assert plan.algo_name == "winograd_half" and plan.n_tiles == n
    y = cn.conv3d(_dev(x), _dev(wt), **case.conv_kwargs(), algo="winograd_half", out=poisoned(yr.shape, x.dtype))
    err = check_parity(y.cpu(), yr, den, y.dtype, case.name)
    assert err < WH_BOUND[y.dtype], err


def test_winograd_half_scales_follow_the_data():
    """One workspace, inputs of very different magnitudes in turn: each call
    picks its own scales (nothing carries over), so each result equals a fresh
    run's bits and scales with the input exactly."""
    case = cw.ConvCase("wh_rescale", 2, 20, 22, 64, 48, 3, 3, (1, 1), (1, 1), (1, 1), "bf16", "normal", "normal",
                       None, 66, 0)
    x, w = _dev(case.input()), _dev(case.weight())
    plan = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, torch.bfloat16, algo="winograd_half")
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    outs = {}
    for scale in (2.0 ** 40, 1.0, 2.0 ** -40, 1.0):
        xs = x * scale  # exact: a power of two
        y = cn.conv2d(xs, w, 1, 1, 1, plan=plan, workspace=ws)
        fresh = cn.conv2d(xs, w, 1, 1, 1, algo="winograd_half")
        assert torch.equal(bits(y), bits(fresh)), scale
        outs[scale] = y
    # power-of-two input scales move only the scale exponents: the same bits, rescaled
    assert torch.equal(bits(outs[2.0 ** 40] * 2.0 ** -40), bits(outs[1.0]))
    assert torch.equal(bits(outs[2.0 ** -40] * 2.0 ** 40), bits(outs[1.0]))


def test_winograd_half_3d_kd1_bit_identical_to_conv2d():
    """KD = 1: the 3D path is the 2D path over the frames, bit for bit."""
    case = cw.ConvCase("wh3d_vs_2d", 1, 12, 14, 64, 48, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), "f16", "normal",
                       "normal", None, 65, 0, nd=3, d=5, kd=1)
    x, wt = _dev(case.input()), _dev(case.weight())
    y3 = cn.conv3d(x, wt, **case.conv_kwargs(), algo="winograd_half")
    y2 = cn.conv2d(x[0], wt[:, 0], 1, 1, 1, algo="winograd_half")
    assert torch.equal(bits(y3[0]), bits(y2))
