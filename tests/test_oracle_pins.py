"""Pins for the CPU oracle (no GPU).

The oracle is trusted only because of these tests.  Each pin comes from outside
the oracle's own code:
  * brute force: tests/brute.py, pure-Python loops, exact on integer data;
  * a library convolution: torch.nn.functional.conv2d / conv3d in float64 on
    the CPU, and scipy.signal.correlate2d for single-channel cases;
  * closed forms: a 1x1 stride-1 conv is a matmul; a delta input reproduces
    the (spatially flipped) weights;
  * invariants: linearity in x and in w; 3D = sum over depth taps of 2D convs
    on frame views (the decomposition of the small-kernel-depth page, section
    Change); output-row subsets equal the matching rows of the full output.
A plausible mistake in the oracle -- a dropped tap, a sign or index slip in the
input coordinate, swapped kh/kw, transposed weights, an off-by-one in the output
extent -- fails at least the brute-force and library pins.
"""
import itertools

import numpy as np
import pytest
import scipy.signal
import torch
import torch.nn.functional as F

import brute
import oracle


def _tiny_int(rng, shape):
    return rng.integers(-3, 4, size=shape).astype(np.float32)


GEOMS = [(k, s, d, p) for k in (1, 3, 5, 7) for s in (1, 2) for d in (1, 2) for p in (0, 1, 2)
         if not (k == 1 and d == 2)]


@pytest.mark.parametrize("k,s,d,p", GEOMS)
def test_oracle_equals_bruteforce_2d(k, s, d, p):
    rng = np.random.default_rng([11, k, s, d, p])
    h = max(d * (k - 1) + 1 - 2 * p, 1) + 2
    w_ = h + 1
    x = _tiny_int(rng, (2, h, w_, 3))
    wt = _tiny_int(rng, (4, k, k, 3))
    y, den = oracle.conv(x, wt, s, p, d)
    yb = np.array(brute.conv2d(x.astype(int).tolist(), wt.astype(int).tolist(), (s, s), (p, p), (d, d)),
                  dtype=np.float64)
    db = np.array(brute.conv2d(np.abs(x).astype(int).tolist(), np.abs(wt).astype(int).tolist(),
                               (s, s), (p, p), (d, d)), dtype=np.float64)
    assert y.shape == yb.shape
    assert np.array_equal(y, yb)
    assert np.array_equal(den, db)


def test_oracle_equals_bruteforce_asymmetric():
    rng = np.random.default_rng(5)
    x = _tiny_int(rng, (1, 7, 6, 2))
    wt = _tiny_int(rng, (3, 3, 2, 2))
    y, _ = oracle.conv(x, wt, (2, 1), (1, 0), (1, 2))
    yb = brute.conv2d(x.astype(int).tolist(), wt.astype(int).tolist(), (2, 1), (1, 0), (1, 2))
    assert np.array_equal(y, np.array(yb, dtype=np.float64))


@pytest.mark.parametrize("kd,sd,pd", [(1, 1, 0), (2, 1, 0), (3, 1, 0), (3, 2, 1), (5, 1, 0)])
def test_oracle_equals_bruteforce_3d(kd, sd, pd):
    rng = np.random.default_rng([12, kd, sd, pd])
    x = _tiny_int(rng, (1, kd + 2, 4, 5, 2))
    wt = _tiny_int(rng, (3, kd, 3, 3, 2))
    y, den = oracle.conv(x, wt, (sd, 1, 1), (pd, 1, 1), 1)
    yb = brute.conv3d(x.astype(int).tolist(), wt.astype(int).tolist(), (sd, 1, 1), (pd, 1, 1), (1, 1, 1))
    assert np.array_equal(y, np.array(yb, dtype=np.float64))
    db = brute.conv3d(np.abs(x).astype(int).tolist(), np.abs(wt).astype(int).tolist(),
                      (sd, 1, 1), (pd, 1, 1), (1, 1, 1))
    assert np.array_equal(den, np.array(db, dtype=np.float64))


@pytest.mark.parametrize("k,s,d,p", [(3, 1, 1, 1), (5, 2, 1, 2), (7, 2, 2, 0), (3, 2, 2, 1), (1, 2, 1, 0)])
def test_oracle_matches_torch_conv2d_fp64(k, s, d, p):
    rng = np.random.default_rng([13, k, s, d, p])
    x = rng.standard_normal((2, 19, 17, 24)).astype(np.float32)
    wt = rng.standard_normal((20, k, k, 24)).astype(np.float32)
    y, den = oracle.conv(x, wt, s, p, d)
    ref = F.conv2d(torch.from_numpy(x).double().permute(0, 3, 1, 2), torch.from_numpy(wt).double().permute(0, 3, 1, 2),
                   stride=s, padding=p, dilation=d).permute(0, 2, 3, 1).numpy()
    assert y.shape == ref.shape
    assert np.all(np.abs(y - ref) <= 1e-12 * den + 1e-300)


@pytest.mark.parametrize("k,s,d,p", [(3, 1, 1, 1), (3, 2, 1, 1), (5, 1, 2, 4), (1, 1, 1, 0)])
def test_oracle_conv1d_as_h1_matches_torch_conv1d_fp64(k, s, d, p):
    """conv1d through the 2D definition with H = KH = 1 equals torch's conv1d."""
    rng = np.random.default_rng([15, k, s, d, p])
    x = rng.standard_normal((2, 37, 20)).astype(np.float32)
    wt = rng.standard_normal((12, k, 20)).astype(np.float32)
    y, den = oracle.conv(x[:, None], wt[:, None], (1, s), (0, p), (1, d))
    ref = F.conv1d(torch.from_numpy(x).double().permute(0, 2, 1), torch.from_numpy(wt).double().permute(0, 2, 1),
                   stride=s, padding=p, dilation=d).permute(0, 2, 1).numpy()
    assert y[:, 0].shape == ref.shape
    assert np.all(np.abs(y[:, 0] - ref) <= 1e-12 * den[:, 0] + 1e-300)


def test_oracle_matches_torch_conv3d_fp64():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((2, 6, 9, 8, 16)).astype(np.float32)
    wt = rng.standard_normal((12, 3, 3, 3, 16)).astype(np.float32)
    y, den = oracle.conv(x, wt, (1, 2, 1), (0, 1, 2), (1, 1, 2))
    ref = F.conv3d(torch.from_numpy(x).double().permute(0, 4, 1, 2, 3),
                   torch.from_numpy(wt).double().permute(0, 4, 1, 2, 3),
                   stride=(1, 2, 1), padding=(0, 1, 2), dilation=(1, 1, 2)).permute(0, 2, 3, 4, 1).numpy()
    assert y.shape == ref.shape
    assert np.all(np.abs(y - ref) <= 1e-12 * den + 1e-300)


def test_single_channel_equals_scipy_correlate2d():
    rng = np.random.default_rng(15)
    img = rng.standard_normal((13, 11)).astype(np.float32)
    ker = rng.standard_normal((3, 5)).astype(np.float32)
    y, _ = oracle.conv(img[None, :, :, None], ker[None, :, :, None], 1, (1, 2), 1)
    ref = scipy.signal.correlate2d(img.astype(np.float64), ker.astype(np.float64), mode="same")
    assert np.allclose(y[0, :, :, 0], ref, rtol=0, atol=1e-12)


def test_1x1_is_matmul():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((3, 5, 7, 33)).astype(np.float32)
    wt = rng.standard_normal((21, 1, 1, 33)).astype(np.float32)
    y, den = oracle.conv(x, wt, 1, 0, 1)
    ref = x.reshape(-1, 33).astype(np.float64) @ wt.reshape(21, 33).T.astype(np.float64)
    assert np.all(np.abs(y.reshape(-1, 21) - ref) <= 1e-13 * den.reshape(-1, 21))


def test_delta_input_reproduces_flipped_weights():
    rng = np.random.default_rng(17)
    kh, kw, c, o, p = 3, 5, 4, 6, 2
    wt = rng.standard_normal((o, kh, kw, c)).astype(np.float32)
    x = np.zeros((1, 9, 9, c), np.float32)
    h0, w0, c0 = 4, 4, 2
    x[0, h0, w0, c0] = 1.0
    y, _ = oracle.conv(x, wt, 1, p, 1)
    # correlation: y[h0 + p - a, w0 + p - b, o] = w[o, a, b, c0]
    for a, b in itertools.product(range(kh), range(kw)):
        assert np.array_equal(y[0, h0 + p - a, w0 + p - b, :], wt[:, a, b, c0].astype(np.float64))
    mask = np.ones(y.shape[1:3], bool)
    for a, b in itertools.product(range(kh), range(kw)):
        mask[h0 + p - a, w0 + p - b] = False
    assert np.all(y[0][mask] == 0)


def test_linearity_in_x_and_w():
    rng = np.random.default_rng(18)
    x1 = _tiny_int(rng, (1, 8, 8, 5))
    x2 = _tiny_int(rng, (1, 8, 8, 5))
    w1 = _tiny_int(rng, (4, 3, 3, 5))
    w2 = _tiny_int(rng, (4, 3, 3, 5))
    a = lambda x, w: oracle.conv(x, w, 2, 1, 1)[0]
    assert np.array_equal(a(x1 + 2 * x2, w1), a(x1, w1) + 2 * a(x2, w1))
    assert np.array_equal(a(x1, w1 - 3 * w2), a(x1, w1) - 3 * a(x1, w2))


@pytest.mark.parametrize("h,k,s,p,d", [(16, 3, 1, 1, 1), (15, 7, 2, 3, 1), (9, 3, 2, 0, 2), (5, 5, 1, 0, 1),
                                       (224, 7, 2, 3, 1), (7, 1, 2, 0, 1)])
def test_output_shape_formula(h, k, s, p, d):
    ref = F.conv2d(torch.zeros(1, 1, h, h + 3), torch.zeros(1, 1, k, k), stride=s, padding=p, dilation=d).shape
    assert oracle.out_shape((h, h + 3), (k, k), s, p, d) == tuple(ref[2:])


def test_invalid_geometry_rejected():
    with pytest.raises(ValueError):
        oracle.out_shape((2, 2), (5, 5), 1, 0, 1)
    with pytest.raises(ValueError):
        oracle.out_shape((4, 4), (3, 3), 0, 0, 1)


def test_3d_equals_sum_of_2d_over_depth_taps():
    rng = np.random.default_rng(19)
    kd, d = 3, 7
    x = rng.standard_normal((1, d, 6, 5, 16)).astype(np.float32)
    wt = rng.standard_normal((8, kd, 3, 3, 16)).astype(np.float32)
    y3, den3 = oracle.conv(x, wt, 1, (0, 1, 1), 1)
    od = d - kd + 1
    acc = np.zeros_like(y3[0])
    for t in range(kd):
        yt, _ = oracle.conv(x[0, t:t + od], wt[:, t], 1, 1, 1)
        acc += yt
    assert np.all(np.abs(y3[0] - acc) <= 1e-13 * den3[0])


def test_row_subset_matches_full():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((3, 10, 9, 7)).astype(np.float32)
    wt = rng.standard_normal((5, 3, 3, 7)).astype(np.float32)
    yf, df = oracle.conv(x, wt, 1, 1, 1)
    rows = np.array([0, 5, 89, 100, 269], np.int64)
    ys, ds = oracle.conv(x, wt, 1, 1, 1, rows=rows)
    assert np.array_equal(ys, yf.reshape(-1, 5)[rows])
    assert np.array_equal(ds, df.reshape(-1, 5)[rows])
    with pytest.raises(ValueError):
        oracle.conv(x, wt, 1, 1, 1, rows=np.array([270], np.int64))


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 12, 12, 9)).astype(np.float32)
    wt = rng.standard_normal((7, 3, 3, 9)).astype(np.float32)
    y1, _ = oracle.conv(x, wt, 1, 1, 1, threads=1)
    y5, _ = oracle.conv(x, wt, 1, 1, 1, threads=5)
    assert np.array_equal(y1, y5)
