"""Planner tests (host logic only, no GPU): cnhwc_conv_select and the Winograd
batch-tiling rule, including the memory figures printed on MLX PR "Bound
winograd conv2d working set by tiling the batch" (tests/golden/tiling_page_memory.txt).
"""
import ctypes
import math
import os

import pytest
import torch

import convolution_nhwc_conv2d_amd as cn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiling_page_memory.txt")
GB = 1e9


def _golden():
    rows = {"m4pro": [], "m2max": [], "m5max_elements": None, "m5max_peak": None}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "m4pro":
            rows["m4pro"].append((int(line[1]), float(line[2]), float(line[3])))
        elif line[0] == "m2max":
            rows["m2max"].append((int(line[1]), float(line[2]), float(line[3])))
        elif line[0] == "m5max_elements":
            rows["m5max_elements"] = int(line[1])
        elif line[0] == "m5max_peak":
            rows["m5max_peak"] = (float(line[1]), float(line[2]))
    return rows


# ---- the buffer set the tiling page describes for MLX's Winograd (Problem):
# padded input + input-transform GEMM operand V + GEMM result M per element,
# and the conv's own tensors x, y, transformed filter U (Fix).
def _mlx_buffers(h, w, c, o, m):
    """Bytes per batch element for F(m x m, 3x3) (fp32): x, y, pad, V, M; and U."""
    t = m + 2
    th, tw = math.ceil(h / m), math.ceil(w / m)
    tiles = th * tw
    x = h * w * c * 4
    y = h * w * o * 4
    pad = (th * m + 2) * (tw * m + 2) * c * 4  # padded to whole tiles plus the 2-pixel halo
    v = t * t * tiles * c * 4
    mm = t * t * tiles * o * 4
    u = t * t * o * c * 4
    return x, y, pad, v, mm, u, tiles


def test_golden_untiled_peaks_single_out_f6x3():
    """The control peaks (no tiling) are reproduced only by 8x8 tiles at stride 6."""
    g = _golden()
    for m, expect in ((6, True), (4, False), (2, False)):
        x, y, pad, v, mm, u, _ = _mlx_buffers(512, 512, 192, 96, m)
        ok = all(round((n * (x + y + pad + v + mm) + u) / GB, 1) == peak for n, peak, _ in g["m4pro"])
        assert ok == expect, m
    x, y, pad, v, mm, u, _ = _mlx_buffers(512, 512, 192, 96, 6)
    for n, untiled, _ in g["m2max"]:
        assert round((n * (x + y + pad + v + mm) + u) / GB) == untiled


def test_golden_tiled_peaks_follow_the_budget_rule():
    """Some single working-set figure W gives all four printed M4 Pro tiled peaks
    through the rule tile = min(N, floor((3/4 W - own) / scratch))."""
    g = _golden()
    x, y, pad, v, mm, u, tiles = _mlx_buffers(512, 512, 192, 96, 6)
    scratch = pad + v + mm
    hits = []
    for wmb in range(39000, 42000, 5):
        wl = wmb * 10**6
        tiles_ok = []
        for n, _, tiled in g["m4pro"]:
            own = n * (x + y) + u
            tb, _, fb = cn.winograd_tile_rule(wl, own, scratch, n, tiles)
            if fb or round((own + tb * scratch) / GB, 1) != tiled:
                break
            tiles_ok.append(tb)
        else:
            hits.append((wl, tuple(tiles_ok)))
    assert hits, "no W reproduces the printed tiled peaks"
    assert {t for _, t in hits} == {(27, 24, 20, 14)}
    assert 40.1e9 < min(w for w, _ in hits) and max(w for w, _ in hits) < 40.4e9
    # M2 Max, batch 80: the printed tiled peak is the tile of 45 elements
    for n, _, tiled in g["m2max"]:
        own = n * (x + y) + u
        assert [tb for tb in range(1, n) if round((own + tb * scratch) / GB) == tiled] == [45]


def test_golden_injected_512mb_case():
    """N=16, 128x128, 192->96 is the shape whose output has the printed element
    count; at an injected 512 MB budget the rule gives one-element tiles and the
    printed 0.36 GB peak, and at 1 MB it falls back."""
    g = _golden()
    assert 16 * 128 * 128 * 96 == g["m5max_elements"]
    x, y, pad, v, mm, u, tiles = _mlx_buffers(128, 128, 192, 96, 6)
    own = 16 * (x + y) + u
    untiled = 16 * (x + y + pad + v + mm) + u
    assert round(untiled / GB, 2) == g["m5max_peak"][0]
    for wl in (512 * 10**6, 512 * 2**20):
        tb, _, fb = cn.winograd_tile_rule(wl, own, pad + v + mm, 16, tiles)
        assert (tb, fb) == (1, False)
        assert round((own + tb * (pad + v + mm)) / GB, 2) == g["m5max_peak"][1]
    tb, _, fb = cn.winograd_tile_rule(2**20, own, pad + v + mm, 16, tiles)
    assert fb and tb == 0


# ------------------------------------------------------------ our own plans

def _p(xs, ws, stride=1, pad=1, dil=1, dtype=torch.float32, **kw):
    return cn.plan2d(xs, ws, stride, pad, dil, dtype, **kw)


C2W = (96, 3, 3, 192)


def test_wide_fp32_full_budget_is_untiled_winograd():
    p = _p((40, 512, 512, 192), C2W, ws_limit=288 * 10**9)
    assert p.algo_name == "winograd" and p.tile_batch == 40 and p.n_tiles == 1
    assert p.tiles_per_image == 86 * 86
    # V + M + the tile masks (192 channel threads per tile: three 8-byte parts)
    assert p.scratch_per_element == 64 * 7396 * (192 + 96) * 4 + 7396 * 3 * 8
    # x + y + U + the tap masks (one 32-bit word per output channel)
    assert p.own_bytes == 40 * 512 * 512 * (192 + 96) * 4 + 64 * 96 * 192 * 4 + 96 * 4
    assert p.workspace_bytes >= 64 * 96 * 192 * 4 + 40 * p.scratch_per_element
    assert p.budget_bytes == 288 * 10**9 // 4 * 3 - p.own_bytes


@pytest.mark.parametrize("n", [8, 32, 40, 64])
@pytest.mark.parametrize("wl", [512 * 10**6, 512 * 2**20, 10**6, 2**20])
def test_wide_fp32_small_budgets_fall_back(n, wl):
    p = _p((n, 512, 512, 192), C2W, ws_limit=wl)
    assert p.algo_name == "implicit_gemm" and p.workspace_bytes == 0


@pytest.mark.parametrize("n", [32, 40, 48, 64])
def test_wide_fp32_m4pro_class_budget_tiles(n):
    wl = 40_200_000_000
    p = _p((n, 512, 512, 192), C2W, ws_limit=wl)
    own = n * 512 * 512 * (192 + 96) * 4 + 64 * 96 * 192 * 4 + 96 * 4
    scratch = 64 * 7396 * (192 + 96) * 4 + 7396 * 3 * 8
    tb = min(n, (wl * 3 // 4 - own) // scratch)
    assert p.algo_name == "winograd" and p.tile_batch == tb and p.n_tiles == -(-n // tb)


def test_page_shape_512mib_tiles_our_scratch():
    p = _p((16, 128, 128, 192), C2W, ws_limit=512 * 2**20)
    assert p.algo_name == "winograd" and p.tile_batch == 2 and p.n_tiles == 8
    assert _p((16, 128, 128, 192), C2W, ws_limit=2**20).algo_name == "implicit_gemm"


def test_forced_tile_is_capped_by_budget_and_leaves_short_final_tile():
    p = _p((40, 512, 512, 192), C2W, ws_limit=40_200_000_000, tile_batch=1000)
    q = _p((40, 512, 512, 192), C2W, ws_limit=40_200_000_000)
    assert p.tile_batch == q.tile_batch
    p = _p((40, 512, 512, 192), C2W, tile_batch=3)
    assert p.tile_batch == 3 and p.n_tiles == 14  # 13 tiles of 3 and a final tile of 1
    p = _p((40, 512, 512, 192), C2W, tile_batch=7)
    assert p.tile_batch == 7 and p.n_tiles == 6


def test_min_tile_rows_fallback_for_spatially_tiny_convs():
    # the page's 256 x 4x4, 64 -> 192 conv: one 6x6 tile per image
    xs, ws = (256, 4, 4, 64), (192, 3, 3, 64)
    assert _p(xs, ws).algo_name == "winograd"  # whole batch fits: unchanged
    full = _p(xs, ws, ws_limit=10**12)
    wl = -(-(full.own_bytes + 100 * full.scratch_per_element) * 4 // 3)
    p = _p(xs, ws, ws_limit=wl)
    assert p.algo_name == "implicit_gemm"  # 100 one-tile elements = 100 rows < 256
    p = _p(xs, ws, ws_limit=wl, tile_batch=50)
    assert p.algo_name == "winograd" and p.tile_batch == 50  # a forced tile bypasses the floor


@pytest.mark.parametrize("c,o,dtype,expect", [
    (192, 96, torch.float32, "winograd"), (160, 96, torch.float32, "winograd"),
    (128, 96, torch.float32, "implicit_gemm"), (200, 96, torch.float32, "implicit_gemm"),
    (192, 100, torch.float32, "implicit_gemm"), (256, 256, torch.float16, "implicit_gemm"),
    (256, 512, torch.float16, "implicit_gemm"), (256, 4096, torch.bfloat16, "implicit_gemm"),
    (256, 4096, torch.float32, "winograd")])
def test_auto_gate(c, o, dtype, expect):
    assert _p((2, 32, 32, c), (o, 3, 3, c), dtype=dtype).algo_name == expect


def test_winograd_gate_needs_3x3_stride1_dilation1():
    for xs, ws, s, d in (((1, 32, 32, 192), (96, 3, 3, 192), 2, 1), ((1, 32, 32, 192), (96, 3, 3, 192), 1, 2),
                         ((1, 32, 32, 192), (96, 5, 5, 192), 1, 1)):
        assert _p(xs, ws, s, 1, d).algo_name == "implicit_gemm"
        with pytest.raises(cn.CnhwcError) as e:
            _p(xs, ws, s, 1, d, algo="winograd")
        assert e.value.name == "NOT_APPLICABLE"


def test_forced_winograd_over_budget():
    with pytest.raises(cn.CnhwcError) as e:
        _p((8, 512, 512, 192), C2W, algo="winograd", ws_limit=2**20)
    assert e.value.name == "BUDGET"


def test_unfold_rows_cap_and_forced_rows():
    xs, ws = (16, 32, 32, 256), (1024, 3, 3, 256)
    p = _p(xs, ws, dtype=torch.float16, algo="unfold_gemm")
    k = 9 * 256
    assert p.algo_name == "unfold_gemm"
    assert p.unfold_rows == min(16 * 1024, (256 << 20) // (k * 2))
    assert p.workspace_bytes >= p.unfold_rows * k * 2
    p = _p(xs, ws, dtype=torch.float16, algo="unfold_gemm", unfold_rows=1000)
    assert p.unfold_rows == 1000 and p.n_chunks == 17  # 16 x 1000 + a short chunk of 384


def test_kernel_config_depends_on_channels_and_dtype_only():
    a = _p((40, 512, 512, 192), C2W)
    b = _p((1, 64, 64, 192), C2W, algo="winograd")
    c = _p((40, 512, 512, 192), C2W, ws_limit=40_200_000_000)
    assert a.kernel_config == b.kernel_config == c.kernel_config


def test_select_is_deterministic_bytes():
    d = cn.make_desc((40, 512, 512, 192), C2W, 1, 1, 1, torch.float32)
    o = cn.make_opts(ws_limit=40_200_000_000)
    a, b = cn.select(d, o), cn.select(d, o)
    assert ctypes.string_at(ctypes.addressof(a), ctypes.sizeof(a)) == \
        ctypes.string_at(ctypes.addressof(b), ctypes.sizeof(b))


@pytest.mark.parametrize("xs,ws,s,p,d,err", [
    ((1, 2, 2, 8), (8, 5, 5, 8), 1, 0, 1, "INVALID_ARGUMENT"),   # output extent < 1
    ((1, 8, 8, 8), (8, 3, 3, 8), 0, 0, 1, "INVALID_ARGUMENT"),   # stride 0
    ((1, 8, 8, 8), (8, 3, 3, 8), 1, -1, 1, "INVALID_ARGUMENT"),  # negative pad
    ((0, 8, 8, 8), (8, 3, 3, 8), 1, 0, 1, "INVALID_ARGUMENT"),   # empty batch
])
def test_invalid_descriptors(xs, ws, s, p, d, err):
    with pytest.raises(cn.CnhwcError) as e:
        _p(xs, ws, s, p, d)
    assert e.value.name == err


SPAN = 2**30  # largest in + 2 * pad per axis, and largest C, the 32-bit gathers index


@pytest.mark.parametrize("axis", ["h", "w"])
def test_spatial_span_bound_both_sides(axis):
    """in + 2 * pad up to 2^30 plans; one more is UNSUPPORTED (the gathers hold
    window origins and tap offsets in 32-bit integers)."""
    def shapes(n_in, k):
        return ((1, 1, n_in, 1), (1, 1, k, 1)) if axis == "w" else ((1, n_in, 1, 1), (1, k, 1, 1))
    pad = (0, 1) if axis == "w" else (1, 0)
    xs, ws = shapes(SPAN - 2, 3)
    p = _p(xs, ws, 1, pad, 1, algo="implicit_gemm")
    assert (p.out_w if axis == "w" else p.out_h) == SPAN - 2
    xs, ws = shapes(SPAN - 1, 3)
    with pytest.raises(cn.CnhwcError) as e:
        _p(xs, ws, 1, pad, 1)
    assert e.value.name == "UNSUPPORTED"
    # a long dilated filter whose span reaches past 2^31 in 32 bits
    xs, ws = shapes(2**31, 2049)
    dil = (1, 2**20) if axis == "w" else (2**20, 1)
    with pytest.raises(cn.CnhwcError) as e:
        _p(xs, ws, 1, pad, dil)
    assert e.value.name == "UNSUPPORTED"


def test_depth_and_channel_span_bounds():
    ok = cn.plan3d((1, SPAN - 4, 1, 1, 1), (1, 3, 1, 1, 1), 1, (2, 0, 0), 1, torch.float16, algo="implicit_gemm")
    assert ok.out_d == SPAN - 2
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan3d((1, SPAN - 3, 1, 1, 1), (1, 3, 1, 1, 1), 1, (2, 0, 0), 1, torch.float16)
    assert e.value.name == "UNSUPPORTED"
    assert _p((1, 1, 1, SPAN), (1, 1, 1, SPAN), 1, 0, 1, algo="implicit_gemm").algo_name == "implicit_gemm"
    with pytest.raises(cn.CnhwcError) as e:
        _p((1, 1, 1, SPAN + 1), (1, 1, 1, SPAN + 1), 1, 0, 1)
    assert e.value.name == "UNSUPPORTED"


def test_invalid_opts_and_groups():
    d = cn.make_desc((1, 8, 8, 8), (8, 3, 3, 8), 1, 1, 1)
    with pytest.raises(cn.CnhwcError) as e:
        cn.select(d, cn.make_opts(ws_limit=0))
    assert e.value.name == "INVALID_ARGUMENT"
    d.groups = 2
    with pytest.raises(cn.CnhwcError) as e:
        cn.select(d, cn.make_opts())
    assert e.value.name == "UNSUPPORTED"


# ------------------------------------------------------------------- 3D

X3, W3 = (1, 41, 60, 104, 256), (256, 3, 3, 3, 256)


def test_3d_video_shapes_take_the_half_winograd():
    """bf16 video shapes: AUTO runs the half-precision Winograd path with the
    depth taps summed in its GEMMs (rule 1b: KD C = 768 or 1536); the native 3D
    GEMM and the decomposition stay available when forced."""
    for t, h, w, c, o in ((17, 64, 64, 256, 256), (41, 60, 104, 256, 256), (41, 120, 208, 512, 512)):
        p = cn.plan3d((1, t, h, w, c), (o, 3, 3, 3, c), 1, (0, 1, 1), 1, torch.bfloat16)
        assert p.algo_name == "winograd_half" and p.out_d == t - 2 and p.n_tiles == 1
        n = cn.plan3d((1, t, h, w, c), (o, 3, 3, 3, c), 1, (0, 1, 1), 1, torch.bfloat16, algo="implicit_gemm")
        assert n.algo_name == "implicit_gemm"
        q = cn.plan3d((1, t, h, w, c), (o, 3, 3, 3, c), 1, (0, 1, 1), 1, torch.bfloat16, algo="small_kd")
        assert q.algo_name == "small_kd" and q.inner_algo_name in ("implicit_gemm", "unfold_gemm")
        assert q.workspace_bytes >= (t - 2) * h * w * o * 4  # fp32 accumulator
    # channels too few for rule 1b (KD C = 192): the native 3D GEMM
    p = cn.plan3d((1, 17, 64, 64, 64), (128, 3, 3, 3, 64), 1, (0, 1, 1), 1, torch.bfloat16)
    assert p.algo_name == "implicit_gemm"


def test_3d_fp32_decomposes_for_winograd():
    """fp32 frames pass the 2D Winograd gate: AUTO keeps the decomposition."""
    p = cn.plan3d((1, 9, 64, 64, 128), (128, 3, 3, 3, 128), 1, (0, 1, 1), 1, torch.float32)
    assert p.algo_name == "small_kd" and p.inner_algo_name == "winograd"


# 32 channels: below rule 1b's KD C >= 384 for every change below, so the
# decomposition guard alone decides.
X3G, W3G = (1, 9, 20, 24, 32), (32, 3, 3, 3, 32)


@pytest.mark.parametrize("change", ["n2", "kd9", "stride_d", "dil_h", "pad_d", "c_mod16", "o_mod16"])
def test_3d_guard_each_clause(change):
    xs, ws = list(X3G), list(W3G)
    s, p, d = [1, 1, 1], [0, 1, 1], [1, 1, 1]
    if change == "n2":
        xs[0] = 2
    elif change == "kd9":
        ws[1] = 9
    elif change == "stride_d":
        s[0] = 2
    elif change == "dil_h":
        d[1] = 2
    elif change == "pad_d":
        p[0] = 1
    elif change == "c_mod16":
        xs[-1] = ws[-1] = 40
    elif change == "o_mod16":
        ws[0] = 40
    # what the guard rejects falls through to the native 3D GEMM
    assert cn.plan3d(tuple(xs), tuple(ws), s, p, d, torch.bfloat16).algo_name == "implicit_gemm"
    # a forced inner algorithm needs the decomposition, so it follows the guard
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan3d(tuple(xs), tuple(ws), s, p, d, torch.bfloat16, inner_algo="implicit_gemm")
    assert e.value.name == "NOT_APPLICABLE"
    structural = change in ("n2", "stride_d", "pad_d")
    if structural:
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan3d(tuple(xs), tuple(ws), s, p, d, torch.bfloat16, algo="small_kd")
        assert e.value.name == "NOT_APPLICABLE"
    else:  # forcing the decomposition only needs its structural conditions
        assert cn.plan3d(tuple(xs), tuple(ws), s, p, d, torch.bfloat16, algo="small_kd").algo_name == "small_kd"


def test_3d_forced_algorithms():
    assert cn.plan3d(X3, W3, 1, (0, 1, 1), 1, torch.bfloat16, algo="implicit_gemm").algo_name == "implicit_gemm"
    for algo in ("winograd", "unfold_gemm"):
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan3d(X3, W3, 1, (0, 1, 1), 1, torch.bfloat16, algo=algo)
        assert e.value.name == "NOT_APPLICABLE"
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan3d(X3, W3, 1, (0, 1, 1), 1, torch.bfloat16, algo="implicit_gemm", inner_algo="implicit_gemm")
    assert e.value.name == "INVALID_ARGUMENT"


def test_3d_forced_inner_winograd():
    p = cn.plan3d(X3, W3, 1, (0, 1, 1), 1, torch.bfloat16, inner_algo="winograd")
    assert p.inner_algo_name == "winograd" and p.tile_batch == 39


# ------------------------------------------------------- GEMM tile choice

F16 = torch.float16


def test_large_half_convs_take_the_256_tiles():
    """Large fp16/bf16 implicit GEMMs of 3x3 stride-1 convs with C % 64 == 0 get
    the patch-staged 256x256 tile (16); other large ones with C % 32 == 0 the
    256x256 direct-to-LDS tile (14); small ones (a ResNet-50 batch-1 layer) and
    C % 32 != 0 neither."""
    big = cn.plan2d((64, 32, 32, 256), (4096, 3, 3, 256), 1, 1, 1, F16, algo="implicit_gemm")
    assert big.kernel_config == 16
    big3 = cn.plan3d((1, 41, 120, 208, 512), (512, 3, 3, 3, 512), 1, (0, 1, 1), 1, torch.bfloat16,
                     algo="implicit_gemm")
    assert big3.kernel_config == 16
    for xs, ws, s in (((64, 32, 32, 96), (4096, 3, 3, 96), 1), ((64, 64, 64, 256), (4096, 3, 3, 256), 2),
                      ((64, 32, 32, 256), (4096, 5, 5, 256), 1)):
        assert cn.plan2d(xs, ws, s, 1, 1, F16, algo="implicit_gemm").kernel_config == 14
    small = cn.plan2d((1, 56, 56, 64), (64, 3, 3, 64), 1, 1, 1, F16)
    assert small.kernel_config not in (14, 16)
    odd = cn.plan2d((64, 32, 32, 120), (4096, 3, 3, 120), 1, 1, 1, F16, algo="implicit_gemm")
    assert odd.kernel_config not in (14, 16)


def test_patch_tile_forcing():
    """Config 16 needs 3x3 taps at stride 1 and dilation 1 in the image plane and
    C % 64 == 0 (any depth geometry); it takes no K split."""
    ok = cn.plan2d((2, 20, 20, 64), (300, 3, 3, 64), 1, 1, 1, F16, algo="implicit_gemm", gemm_config=16)
    assert ok.kernel_config == 16 and ok.split_k == 1 and ok.workspace_bytes == 0
    ok3 = cn.plan3d((2, 8, 17, 15, 64), (256, 3, 3, 3, 64), (2, 1, 1), (1, 1, 1), (2, 1, 1), torch.bfloat16,
                    algo="implicit_gemm", gemm_config=16)
    assert ok3.kernel_config == 16
    for xs, ws, s, d, dt in (((2, 20, 20, 96), (64, 3, 3, 96), 1, 1, F16), ((2, 20, 20, 64), (64, 3, 3, 64), 2, 1, F16),
                             ((2, 20, 20, 64), (64, 3, 3, 64), 1, 2, F16), ((2, 20, 20, 64), (64, 5, 5, 64), 1, 1, F16),
                             ((2, 20, 20, 64), (64, 3, 3, 64), 1, 1, torch.float32)):
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan2d(xs, ws, s, 1, d, dt, algo="implicit_gemm", gemm_config=16)
        assert e.value.name == "NOT_APPLICABLE"
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan2d((2, 20, 20, 64), (300, 3, 3, 64), 1, 1, 1, F16, algo="implicit_gemm", gemm_config=16, split_k=2)
    assert e.value.name == "NOT_APPLICABLE"
    with pytest.raises(cn.CnhwcError) as e:  # dense A (unfold rows) never takes it
        cn.plan2d((2, 20, 20, 64), (300, 3, 3, 64), 1, 1, 1, F16, algo="unfold_gemm", gemm_config=16)
    assert e.value.name == "NOT_APPLICABLE"


def test_forced_gemm_config():
    p = cn.plan2d((2, 20, 20, 64), (300, 3, 3, 64), 1, 1, 1, F16, gemm_config=14)
    assert p.kernel_config == 14 and p.opts.force_gemm_config == 14
    p = cn.plan2d((2, 20, 20, 64), (300, 3, 3, 64), 1, 1, 1, F16, algo="unfold_gemm", gemm_config=14)
    assert p.kernel_config == 14
    for xs, ws, dt, algo, cfg in [((2, 20, 20, 64), (300, 3, 3, 64), torch.float32, "implicit_gemm", 14),
                                  ((2, 20, 20, 48), (300, 3, 3, 48), F16, "implicit_gemm", 14),
                                  ((2, 20, 20, 20), (300, 3, 3, 20), F16, "unfold_gemm", 14),
                                  ((2, 20, 20, 64), (300, 3, 3, 64), F16, "implicit_gemm", 3),
                                  ((2, 20, 20, 64), (300, 3, 3, 64), torch.float32, "implicit_gemm", 11),
                                  ((2, 20, 20, 64), (300, 3, 3, 64), F16, "implicit_gemm", 99)]:
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan2d(xs, ws, 1, 1, 1, dt, algo=algo, gemm_config=cfg)
        assert e.value.name == "NOT_APPLICABLE", (xs, dt, algo, cfg)
    d = cn.make_desc((1, 8, 8, 8), (8, 3, 3, 8), 1, 1, 1)
    o = cn.make_opts()
    o.force_gemm_config = -1
    with pytest.raises(cn.CnhwcError) as e:
        cn.select(d, o)
    assert e.value.name == "INVALID_ARGUMENT"
    o = cn.make_opts()
    o.force_split_k = -1
    with pytest.raises(cn.CnhwcError) as e:
        cn.select(d, o)
    assert e.value.name == "INVALID_ARGUMENT"


# ------------------------------------------------------------- split K

def test_split_k_for_small_grids_only():
    """A GEMM grid too small to fill the device splits K; a large one does not."""
    small = cn.plan2d((1, 7, 7, 512), (512, 3, 3, 512), 1, 1, 1, F16)   # ResNet-50 layer4, batch 1
    assert small.split_k > 1
    m, o = 49, 512
    assert small.workspace_bytes == -(-small.split_k * m * o * 4 // 256) * 256
    assert cn.lib.cnhwc_launch_count(ctypes.byref(cn.make_desc((1, 7, 7, 512), (512, 3, 3, 512), 1, 1, 1, F16)),
                                     ctypes.byref(small)) == 2
    big = cn.plan2d((64, 32, 32, 256), (4096, 3, 3, 256), 1, 1, 1, F16)
    assert big.split_k == 1
    wino = cn.plan2d((2, 64, 64, 192), (96, 3, 3, 192), 1, 1, 1, algo="winograd", split_k=4)
    assert wino.split_k == 1


def test_forced_split_k():
    xs, ws = (1, 7, 7, 512), (512, 3, 3, 512)   # K = 4608 = 72 chunks of 64
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, split_k=1).split_k == 1
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, split_k=3).split_k == 3
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, split_k=7).split_k == 7    # 11 chunks per split, last 6
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, split_k=72).split_k == 72
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, split_k=50).split_k == 36  # 2 chunks each: 36 splits
    p = cn.plan2d(xs, ws, 1, 1, 1, F16, algo="unfold_gemm", split_k=5)
    assert p.split_k == 5 and p.workspace_bytes >= 5 * 49 * 512 * 4
    for kw in [dict(split_k=73), dict(split_k=2, gemm_config=14)]:
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan2d(xs, ws, 1, 1, 1, F16, **kw)
        assert e.value.name == "NOT_APPLICABLE", kw


# ------------------------------------- half-precision Winograd F(4x4,3x3)

BF16 = torch.bfloat16
HEAD = 8448  # partial maxima of x and w (2 x 1024 words) + 4 scales, 256-aligned


def _mask_parts(g):
    """8-byte parts of one tile's nonzero-pixel mask for g input-transform
    threads per tile: one per wavefront of 64, else at most one per workgroup
    of 256 that the tile's threads touch."""
    return g // 64 if g % 64 == 0 else (g - 1) // 256 + 2


def _wh_scratch(t, c, o, frames=1, od=1):
    cs = -(-c // 32) * 32
    vec = 4 if c % 4 == 0 else (2 if c % 2 == 0 else 1)
    return 36 * t * (frames * cs * 2 + od * o * 4) + frames * t * _mask_parts(cs // vec) * 8


def test_winograd_half_2d_plan():
    xs, ws = (8, 56, 56, 200), (256, 3, 3, 200)
    p = cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", ws_limit=288 * 10**9)
    t = 14 * 14
    assert p.algo_name == "winograd_half" and p.tiles_per_image == t
    assert p.tile_batch == 8 and p.n_tiles == 1 and p.split_k == 1
    assert p.scratch_per_element == _wh_scratch(t, 200, 256)
    u = 36 * 256 * 224 * 2
    assert p.own_bytes == 8 * 56 * 56 * (200 + 256) * 2 + HEAD + u + 256 * 4  # + the tap masks
    assert p.workspace_bytes >= HEAD + u + 8 * p.scratch_per_element
    assert p.kernel_config in (14, 15)
    desc = cn.make_desc(xs, ws, 1, 1, 1, F16)
    assert cn.lib.cnhwc_launch_count(ctypes.byref(desc), ctypes.byref(p)) == 5
    # ragged output (OH = 53 -> 14 tile rows), padding 0, bf16
    q = cn.plan2d((3, 55, 57, 64), (96, 3, 3, 64), 1, 0, 1, BF16, algo="winograd_half")
    assert q.out_h == 53 and q.out_w == 55 and q.tiles_per_image == 14 * 14


def test_winograd_half_geometry_gate():
    xs = (2, 32, 32, 64)
    for ws, kw in [((64, 3, 3, 64), dict(dtype=torch.float32)),
                   ((64, 5, 5, 64), dict(dtype=F16)),
                   ((64, 3, 3, 64), dict(dtype=F16, stride=2)),
                   ((64, 3, 3, 64), dict(dtype=F16, dil=2)),
                   ((64, 3, 3, 64), dict(dtype=F16, pad=2)),       # corner windows mostly padding
                   ((64, 3, 3, 64), dict(dtype=F16, pad=(1, 2)))]:
        dt = kw.pop("dtype")
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan2d(xs, ws, kw.get("stride", 1), kw.get("pad", 1), kw.get("dil", 1), dt, algo="winograd_half")
        assert e.value.name == "NOT_APPLICABLE", (ws, dt, kw)
    with pytest.raises(cn.CnhwcError) as e:                  # too few channels to average rounding
        cn.plan2d((2, 32, 32, 15), (64, 3, 3, 15), 1, 1, 1, F16, algo="winograd_half")
    assert e.value.name == "NOT_APPLICABLE"
    assert cn.plan2d((2, 32, 32, 16), (64, 3, 3, 16), 1, 1, 1, F16, algo="winograd_half").algo_name == "winograd_half"
    assert cn.plan2d(xs, (64, 3, 3, 64), 1, 0, 1, F16, algo="winograd_half").algo_name == "winograd_half"


@pytest.mark.parametrize("xs,ws,pad,expect", [
    ((16, 32, 32, 512), (512, 3, 3, 512), 1, True),     # 1024 GEMM rows, C O = 16.5 (11C + 20O)
    ((16, 32, 32, 512), (320, 3, 3, 512), 1, True),     # C O = 13.6 (11C + 20O)
    ((8, 56, 56, 512), (256, 3, 3, 512), 1, False),     # C O = 12.2 (11C + 20O)
    ((16, 28, 28, 384), (384, 3, 3, 384), 1, False),    # C O = 12.4 (11C + 20O)
    ((8, 56, 56, 256), (512, 3, 3, 256), 1, False),     # C = 256 < 384
    ((64, 32, 32, 256), (4096, 3, 3, 256), 1, False),   # C = 256
    ((8, 32, 32, 1024), (4096, 3, 3, 1024), 1, True),   # 512 GEMM rows
    ((8, 14, 14, 512), (512, 3, 3, 512), 1, False),     # 128 GEMM rows
    ((32, 14, 14, 512), (512, 3, 3, 512), 1, True),     # 512 GEMM rows
    ((8, 56, 56, 512), (512, 3, 3, 512), 0, True),
    ((8, 56, 56, 512), (512, 3, 3, 512), 2, False),     # padding 2: not for this path
])
def test_winograd_half_auto_rule(xs, ws, pad, expect):
    for dt in (F16, BF16):
        p = cn.plan2d(xs, ws, 1, pad, 1, dt)
        assert (p.algo_name == "winograd_half") == expect, (xs, ws, dt, p.algo_name)
        if not expect:
            assert p.algo_name == "implicit_gemm"
    assert cn.plan2d(xs, ws, 1, pad, 1, torch.float32).algo_name != "winograd_half"


def test_winograd_half_auto_falls_back_over_budget():
    xs, ws = (16, 32, 32, 512), (512, 3, 3, 512)
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, ws_limit=10**6).algo_name == "implicit_gemm"


def test_winograd_half_gemm_tile_choice():
    """K <= 1152 and O <= 512: the 256x128 tile at two workgroups per CU;
    otherwise the occupancy model (the 256x256 tile on these shapes)."""
    assert cn.plan2d((16, 32, 32, 512), (512, 3, 3, 512), 1, 1, 1, F16).kernel_config == 15
    assert cn.plan2d((16, 32, 32, 1024), (512, 3, 3, 1024), 1, 1, 1, F16).kernel_config == 15
    assert cn.plan2d((16, 32, 32, 512), (1024, 3, 3, 512), 1, 1, 1, F16).kernel_config == 14
    assert cn.plan2d((16, 32, 32, 2048), (512, 3, 3, 2048), 1, 1, 1, F16).kernel_config == 14
    v = cn.plan3d((1, 41, 120, 208, 512), (512, 3, 3, 3, 512), 1, (0, 1, 1), 1, BF16)   # K = 1536
    assert v.algo_name == "winograd_half" and v.kernel_config == 14
    v = cn.plan3d((1, 41, 60, 104, 256), (256, 3, 3, 3, 256), 1, (0, 1, 1), 1, BF16)    # K = 768
    assert v.kernel_config == 15


def test_winograd_half_budget_tiles_and_over_budget():
    xs, ws = (16, 64, 64, 128), (128, 3, 3, 128)
    full = cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", ws_limit=288 * 10**9)
    per = full.scratch_per_element
    wl = (full.own_bytes + 5 * per) * 4 // 3 + 8
    p = cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", ws_limit=wl)
    assert p.tile_batch == 5 and p.n_tiles == 4
    f = cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", ws_limit=wl, tile_batch=3)
    assert f.tile_batch == 3 and f.n_tiles == 6
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", ws_limit=10**6)
    assert e.value.name == "BUDGET"


def test_winograd_half_forced_gemm_tiles():
    xs, ws = (4, 32, 32, 64), (96, 3, 3, 64)
    for cfg in (14, 15):
        assert cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", gemm_config=cfg).kernel_config == cfg
    for cfg in (11, 3):
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", gemm_config=cfg)
        assert e.value.name == "NOT_APPLICABLE"
    assert cn.plan2d(xs, ws, 1, 1, 1, F16, algo="winograd_half", split_k=4).split_k == 1


def test_winograd_half_3d_plan():
    xs, ws = (2, 9, 20, 24, 64), (80, 3, 3, 3, 64)
    p = cn.plan3d(xs, ws, 1, (1, 1, 1), (2, 1, 1), BF16, algo="winograd_half")
    # depth: 9 frames + 2 pad = 11, dilation 2 -> OD = 11 - 4 = 7
    assert p.algo_name == "winograd_half" and p.out_d == 7 and p.out_h == 20 and p.out_w == 24
    t = 5 * 6
    assert p.tile_batch == 1 and p.n_tiles == 2 and p.tiles_per_image == t
    assert p.scratch_per_element == _wh_scratch(t, 64, 80, frames=11, od=7)
    desc = cn.make_desc(xs, ws, 1, (1, 1, 1), (2, 1, 1), BF16)
    assert cn.lib.cnhwc_launch_count(ctypes.byref(desc), ctypes.byref(p)) == 2 + 3 * 2
    # depth stride 2 and spatial 5x5 are not for this path; inner algorithms neither
    for args in [dict(s=(2, 1, 1), w=ws), dict(s=1, w=(80, 3, 5, 5, 64))]:
        with pytest.raises(cn.CnhwcError) as e:
            cn.plan3d(xs, args["w"], args["s"], 1, 1, BF16, algo="winograd_half")
        assert e.value.name == "NOT_APPLICABLE"
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan3d(xs, ws, 1, 1, 1, BF16, algo="winograd_half", inner_algo="implicit_gemm")
    assert e.value.name == "INVALID_ARGUMENT"
    with pytest.raises(cn.CnhwcError) as e:
        cn.plan3d((1,) + xs[1:], ws, 1, (0, 1, 1), 1, BF16, inner_algo="winograd_half")
    assert e.value.name == "INVALID_ARGUMENT"


def test_small_channel_half_convs_unfold():
    """fp16/bf16 convs with C % 8 != 0 (element-by-element implicit gather) take
    unfold + GEMM under AUTO; fp32 and C % 8 == 0 keep the implicit GEMM."""
    stem = ((8, 224, 224, 3), (64, 7, 7, 3), 2, 3, 1)
    for dt in (F16, BF16):
        assert cn.plan2d(*stem, dt).algo_name == "unfold_gemm"
        assert cn.plan2d((8, 56, 56, 12), (64, 3, 3, 12), 1, 1, 1, dt).algo_name == "unfold_gemm"
        assert cn.plan2d((8, 56, 56, 16), (64, 3, 3, 16), 1, 1, 1, dt).algo_name == "implicit_gemm"
    assert cn.plan2d(*stem, torch.float32).algo_name == "implicit_gemm"
