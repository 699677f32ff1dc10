"""GPU parity at the workloads' full sizes, on seeded output samples.

The oracle computes the sampled output pixels one by one (all output channels
each); the HIP path runs the whole conv in the launch configuration the
benchmark uses.  Workloads (from the MLX pages):
  * fp32 512x512, 192 -> 96, 3x3, batch 8/32/40/64, under the full, an
    M4-Pro-class and the injected 512 MB / 1 MB budgets (MLX PR "Bound winograd
    conv2d working set by tiling the batch", Testing and review);
  * half-precision C_out / K axes, unaligned channels, wide filters with stride
    and dilation (MLX PR "Use the explicit gemm for wide convs on neural
    accelerators", intro tables and Verified);
  * the ResNet-50 conv stack at batch 1 and 8 (same page, ResNet-50 follow-up);
  * bf16 3x3x3 video convs (MLX PR "Decompose small kernel-depth 3D convs into
    2D convs", Results).
"""
import numpy as np
import pytest
import torch

import conv_workloads as cw
import oracle
from gpu_util import bits, check_parity, gather_rows, to_oracle

pytestmark = pytest.mark.gpu

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")


def _rows_for(total, count, seed, per_image=None):
    """Seeded sample plus the first and last rows (and image borders)."""
    r = set(cw.sample_rows(total, count, seed).tolist())
    r.update({0, total - 1})
    if per_image:
        r.update({per_image - 1, min(total - 1, per_image)})
    return np.array(sorted(r), dtype=np.int64)


# ------------------------------------------------------ fp32 wide workload

@pytest.fixture(scope="module")
def wide64():
    case = cw.wide_fp32(64)
    w = case.weight()
    x = torch.empty(case.x_shape(), dtype=torch.float32, device="cuda")
    for i in range(case.n):
        x[i].copy_(case.element(i))
    return case, x, w.to("cuda"), w


def _check_wide_sample(case, y, n, w_cpu, seed):
    elems = sorted(np.random.default_rng(2 + seed).choice(n, 2, replace=False).tolist())
    per = 512 * 512
    local = _rows_for(2 * per, 3000, seed, per)
    xs = torch.stack([case.element(e) for e in elems])
    yr, den = oracle.conv(to_oracle(xs), to_oracle(w_cpu), 1, 1, 1, rows=local)
    glob = np.array([elems[r // per] * per + r % per for r in local], dtype=np.int64)
    return check_parity(gather_rows(y, glob), yr, den, torch.float32, f"wide n={n}")


@pytest.mark.parametrize("n", [8, 32, 40, 64])
def test_wide_fp32_full_budget_winograd(wide64, n):
    case, x, w, w_cpu = wide64
    xn = x[:n]
    p = cn.plan2d(tuple(xn.shape), tuple(w.shape), 1, 1, 1)
    assert p.algo_name == "winograd" and p.n_tiles == 1
    y = cn.conv2d(xn, w, 1, 1, 1)
    assert _check_wide_sample(case, y, n, w_cpu, n) < 2e-5


@pytest.mark.parametrize("n", [8, 64])
@pytest.mark.parametrize("wl", [512 * 10**6, 2**20])
def test_wide_fp32_small_budget_fallback(wide64, n, wl):
    case, x, w, w_cpu = wide64
    xn = x[:n]
    assert cn.plan2d(tuple(xn.shape), tuple(w.shape), 1, 1, 1, ws_limit=wl).algo_name == "implicit_gemm"
    y = cn.conv2d(xn, w, 1, 1, 1, ws_limit=wl)
    assert _check_wide_sample(case, y, n, w_cpu, 100 + n) < 2e-5


def test_wide_fp32_tiled_bit_identical_at_full_size(wide64):
    case, x, w, _ = wide64
    x40 = x[:40]
    full = cn.conv2d(x40, w, 1, 1, 1)
    wl = 40_200_000_000  # an M4-Pro-class working set: the budget forces batch tiles
    p = cn.plan2d(tuple(x40.shape), tuple(w.shape), 1, 1, 1, ws_limit=wl)
    assert p.algo_name == "winograd" and 1 < p.n_tiles and p.tile_batch * (p.n_tiles - 1) < 40
    tiled = cn.conv2d(x40, w, 1, 1, 1, ws_limit=wl)
    assert torch.equal(bits(tiled), bits(full))
    del tiled
    for tb in (1, 7):
        t = cn.conv2d(x[:8], w, 1, 1, 1, tile_batch=tb)
        assert torch.equal(bits(t), bits(full[:8]))


def test_injected_512mib_shape_tiled_bit_identical():
    case = cw.wide_fp32(16, 128, 128)
    x, w = case.input().cuda(), case.weight().cuda()
    full = cn.conv2d(x, w, 1, 1, 1)
    p = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, ws_limit=512 * 2**20)
    assert p.algo_name == "winograd" and p.n_tiles > 1
    tiled = cn.conv2d(x, w, 1, 1, 1, ws_limit=512 * 2**20)
    assert torch.equal(bits(tiled), bits(full))
    fb = cn.conv2d(x, w, 1, 1, 1, ws_limit=2**20)
    yr, den = oracle.conv(to_oracle(case.input()), to_oracle(case.weight()), 1, 1, 1)
    check_parity(fb.cpu(), yr, den, torch.float32, "512mib shape fallback")
    check_parity(full.cpu(), yr, den, torch.float32, "512mib shape winograd")


# ------------------------------------------------------ half-precision sweep

def _half_case(dtype, c_in, c_out, n, k=3, s=1, d=1, p=None, hw=32):
    p = k // 2 * d if p is None else p
    return cw.ConvCase(f"sweep_{dtype}_c{c_in}_o{c_out}_n{n}_k{k}s{s}d{d}", n, hw, hw, c_in, c_out, k, k, (s, s),
                       (p, p), (d, d), dtype, "normal", "normal", None, 3, c_in * 7 + c_out * 3 + n + k * 11 + s + d)


def _check_half(case, algos=("implicit_gemm", "unfold_gemm"), count=512, unfold_rows=None):
    if (case.kh, case.kw, case.stride, case.dil) == (3, 3, (1, 1), (1, 1)) and max(case.pad) <= 1 and case.c >= 16:
        algos = tuple(algos) + ("winograd_half",)
    x, w = case.input(), case.weight()
    xg, wg = x.cuda(), w.cuda()
    p0 = cn.plan2d(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(), dtype=x.dtype)
    total = case.n * p0.out_h * p0.out_w
    rows = _rows_for(total, count, case.case, p0.out_h * p0.out_w)
    yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs(), rows=rows)
    outs = {}
    for a in algos:
        y = cn.conv2d(xg, wg, **case.conv_kwargs(), algo=a, unfold_rows=unfold_rows if a == "unfold_gemm" else None)
        check_parity(gather_rows(y, rows), yr, den, x.dtype, f"{case.name}/{a}")
        outs[a] = y
    return outs


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c_out", [128, 256, 512, 1024, 2048, 4096])
def test_half_cout_axis(dtype, c_out):
    _check_half(_half_case(dtype, 256, c_out, 16))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c_in", [128, 256, 512, 1024])
def test_half_k_axis(dtype, c_in):
    _check_half(_half_case(dtype, c_in, 1024, 16))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c_in,c_out", [(120, 512), (1000, 2048)])
def test_half_unaligned_channels(dtype, c_in, c_out):
    _check_half(_half_case(dtype, c_in, c_out, 16))


@pytest.mark.parametrize("k,s,d,c_out", [(5, 2, 1, 512), (7, 2, 1, 2048), (5, 1, 2, 512), (7, 1, 2, 2048)])
def test_half_wide_filters(k, s, d, c_out):
    _check_half(_half_case("f16", 256, c_out, 8, k, s, d, hw=48))


def test_half_extremes_m65536():
    _check_half(_half_case("bf16", 256, 4096, 64), count=256)
    _check_half(_half_case("f16", 1024, 1024, 64), count=256)


@pytest.mark.parametrize("rows", [1000, 4097])
def test_unfold_chunked_equals_single_chunk(rows):
    case = _half_case("f16", 256, 1024, 16)
    x, w = case.input().cuda(), case.weight().cuda()
    one = cn.conv2d(x, w, 1, 1, 1, algo="unfold_gemm", unfold_rows=16 * 1024)
    chunked = cn.conv2d(x, w, 1, 1, 1, algo="unfold_gemm", unfold_rows=rows)
    p = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, torch.float16, algo="unfold_gemm", unfold_rows=rows)
    assert p.n_chunks == -(-16384 // rows)
    assert torch.equal(bits(one), bits(chunked))


# ------------------------------------------------------------ ResNet-50

@pytest.mark.parametrize("batch", [1, 8])
def test_resnet50_stack(batch):
    for case, _, _ in cw.resnet50_layers(batch):
        x, w = case.input(), case.weight()
        y = cn.conv2d(x.cuda(), w.cuda(), **case.conv_kwargs())
        if batch == 1:
            yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs())
            check_parity(y.cpu(), yr, den, x.dtype, case.name)
        else:
            e = int(np.random.default_rng(case.case).integers(batch))
            yr, den = oracle.conv(to_oracle(x[e:e + 1]), to_oracle(w), **case.conv_kwargs())
            check_parity(y[e:e + 1].cpu(), yr, den, x.dtype, case.name)


# --------------------------------------------------------------------- 3D

@pytest.mark.parametrize("shape", cw.VIDEO3D_SHAPES)
def test_video3d_bf16(shape):
    t, h, w_, c, o = shape
    case = cw.video3d(t, h, w_, c, o)
    x, w = case.input(), case.weight()
    p = cn.plan3d(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(), dtype=x.dtype)
    assert p.algo_name == "winograd_half"  # depth taps summed in the half-precision Winograd GEMMs
    per = p.out_h * p.out_w
    frames = sorted(np.random.default_rng(5).choice(p.out_d, 2, replace=False).tolist())
    rows = np.concatenate([f * per + _rows_for(per, 1024, f) for f in frames]).astype(np.int64)
    yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs(), rows=rows)
    xg, wg = x.cuda(), w.cuda()
    for algo in ("auto", "implicit_gemm", "small_kd"):
        y = cn.conv3d(xg, wg, **case.conv_kwargs(), algo=algo)
        check_parity(gather_rows(y, rows), yr, den, x.dtype, f"{case.name}/{algo}")
        del y


def test_video3d_inner_winograd_variant():
    case = cw.video3d(17, 64, 64, 256, 256)
    x, w = case.input(), case.weight()
    y = cn.conv3d(x.cuda(), w.cuda(), **case.conv_kwargs(), inner_algo="winograd")
    rows = _rows_for(15 * 64 * 64, 2048, 17)
    yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs(), rows=rows)
    check_parity(gather_rows(y, rows), yr, den, x.dtype, "video3d winograd inner")
