"""Exact checks of the Winograd F(6x6,3x3) and F(4x4,3x3) matrices used by the
HIP path (no GPU).

The identity A^T[(G g G^T) * (B^T d B)]A = corr2d(d, g) must hold exactly in
rational arithmetic for every t x t tile d and 3x3 filter g (t = 8 and 6; the
construction in gen_winograd.py).  The headers' floats must be those rationals
rounded to fp32, and the magnitude bounds the half-precision path scales by
must hold (and be attained) for the F(4x4,3x3) transforms.
"""
import os
import re
import sys
from fractions import Fraction as Fr

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_nhwc_conv2d_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_winograd  # noqa: E402


def _mm(a, b):
    return [[sum(a[i][k] * b[k][j] for k in range(len(b))) for j in range(len(b[0]))] for i in range(len(a))]


def _t(a):
    return [list(r) for r in zip(*a)]


def _rand_frac(rng, shape):
    return [[Fr(int(rng.integers(-50, 51)), int(rng.integers(1, 9))) for _ in range(shape[1])] for _ in range(shape[0])]


@pytest.mark.parametrize("m_out", [6, 4])
@pytest.mark.parametrize("seed", range(6))
def test_2d_identity_exact(seed, m_out):
    bt, g, at = gen_winograd.matrices(m_out)
    t = m_out + 2
    rng = np.random.default_rng(seed)
    d = _rand_frac(rng, (t, t))
    f = _rand_frac(rng, (3, 3))
    u = _mm(_mm(g, f), _t(g))
    v = _mm(_mm(bt, d), _t(bt))
    m = [[u[i][j] * v[i][j] for j in range(t)] for i in range(t)]
    y = _mm(_mm(at, m), _t(at))
    ref = [[sum(d[i + a][j + b] * f[a][b] for a in range(3) for b in range(3)) for j in range(m_out)]
           for i in range(m_out)]
    assert y == ref


@pytest.mark.parametrize("m_out", [6, 4])
def test_1d_identity_exact_on_basis(m_out):
    bt, g, at = gen_winograd.matrices(m_out)
    t = m_out + 2
    for p in range(t):
        for q in range(3):
            d = [Fr(int(i == p)) for i in range(t)]
            f = [Fr(int(k == q)) for k in range(3)]
            gu = [sum(g[i][k] * f[k] for k in range(3)) for i in range(t)]
            bv = [sum(bt[i][k] * d[k] for k in range(t)) for i in range(t)]
            y = [sum(at[r][i] * gu[i] * bv[i] for i in range(t)) for r in range(m_out)]
            ref = [sum(d[r + k] * f[k] for k in range(3)) for r in range(m_out)]
            assert y == ref


def test_f43_matches_published_form():
    # The F(4x4,3x3) matrices as Lavin & Gray print them (points 0, +-1, +-2, inf).
    bt, g, at = gen_winograd.matrices(4)
    assert bt[0] == [4, 0, -5, 0, 1, 0]
    assert bt[5] == [0, 4, 0, -5, 0, 1]
    assert g[0] == [Fr(1, 4), 0, 0] and g[5] == [0, 0, 1]
    assert g[3] == [Fr(1, 24), Fr(1, 12), Fr(1, 6)]
    assert at[3] == [0, 1, -1, 8, -8, 1]


def test_f43_magnitude_bounds_hold_and_are_attained():
    """|B^T d B| <= 100 max|d| and |G g G^T| <= max|g|, with equality for the
    sign patterns of the worst rows: the power-of-two scales the half-precision
    kernels pick from these bounds can never overflow fp16, and are not loose."""
    bt, g, at = gen_winograd.matrices(4)
    assert gen_winograd.row_abs_bound(bt) == 10 and gen_winograd.row_abs_bound(g) == 1
    rng = np.random.default_rng(0)
    btf = np.array([[float(e) for e in r] for r in bt])
    gf = np.array([[float(e) for e in r] for r in g])
    for _ in range(200):
        d = rng.uniform(-1, 1, (6, 6))
        assert np.abs(btf @ d @ btf.T).max() <= 100 * np.abs(d).max() + 1e-12
        f = rng.uniform(-1, 1, (3, 3))
        assert np.abs(gf @ f @ gf.T).max() <= np.abs(f).max() + 1e-12
    i = int(np.argmax([sum(abs(e) for e in r) for r in bt]))
    s = np.sign(btf[i])
    d = np.outer(s, s)  # |d| <= 1, hits every term of row i twice
    assert abs((btf @ d @ btf.T)[i, i]) == 100.0
    f = np.ones((3, 3))
    assert abs((gf @ f @ gf.T)[5, 5]) == 1.0


@pytest.mark.parametrize("m_out", [6, 4])
def test_header_matches_rationals_rounded_to_fp32(m_out):
    bt, g, at = gen_winograd.matrices(m_out)
    hdr, names = (("winograd_f63.h", ("kWinoBT", "kWinoG", "kWinoAT")) if m_out == 6
                  else ("winograd_f43.h", ("kWino4BT", "kWino4G", "kWino4AT")))
    text = open(os.path.join(CSRC, hdr)).read()
    for name, mat in zip(names, (bt, g, at)):
        body = re.search(name + r"\[\d+\]\[\d+\] = \{(.*?)\n\};", text, re.S).group(1)
        vals = [float(v) for v in re.findall(r"(-?[0-9.e\-]+)f", body)]
        ref = [float(np.float32(float(e))) for row in mat for e in row]
        assert len(vals) == len(ref)
        assert all(np.float32(a) == np.float32(b) for a, b in zip(vals, ref))
        assert vals == ref
