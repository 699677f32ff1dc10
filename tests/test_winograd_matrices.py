"""Exact checks of the Winograd F(6x6,3x3) matrices used by the HIP path (no GPU).

The identity A^T[(G g G^T) * (B^T d B)]A = corr2d(d, g) must hold exactly in
rational arithmetic for every 8x8 tile d and 3x3 filter g (the construction in
gen_winograd.py).  The header's floats must be those rationals rounded to fp32.
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


@pytest.mark.parametrize("seed", range(6))
def test_2d_identity_exact(seed):
    bt, g, at = gen_winograd.matrices()
    rng = np.random.default_rng(seed)
    d = _rand_frac(rng, (8, 8))
    f = _rand_frac(rng, (3, 3))
    u = _mm(_mm(g, f), _t(g))
    v = _mm(_mm(bt, d), _t(bt))
    m = [[u[i][j] * v[i][j] for j in range(8)] for i in range(8)]
    y = _mm(_mm(at, m), _t(at))
    ref = [[sum(d[i + a][j + b] * f[a][b] for a in range(3) for b in range(3)) for j in range(6)] for i in range(6)]
    assert y == ref


def test_1d_identity_exact_on_basis():
    bt, g, at = gen_winograd.matrices()
    for p in range(8):
        for q in range(3):
            d = [Fr(int(i == p)) for i in range(8)]
            f = [Fr(int(k == q)) for k in range(3)]
            gu = [sum(g[i][k] * f[k] for k in range(3)) for i in range(8)]
            bv = [sum(bt[i][k] * d[k] for k in range(8)) for i in range(8)]
            y = [sum(at[r][i] * gu[i] * bv[i] for i in range(8)) for r in range(6)]
            ref = [sum(d[r + k] * f[k] for k in range(3)) for r in range(6)]
            assert y == ref


def test_header_matches_rationals_rounded_to_fp32():
    bt, g, at = gen_winograd.matrices()
    text = open(os.path.join(CSRC, "winograd_f63.h")).read()
    for name, mat in (("kWinoBT", bt), ("kWinoG", g), ("kWinoAT", at)):
        body = re.search(name + r"\[\d+\]\[\d+\] = \{(.*?)\n\};", text, re.S).group(1)
        vals = [float(v) for v in re.findall(r"(-?[0-9.e\-]+)f", body)]
        ref = [float(np.float32(float(e))) for row in mat for e in row]
        assert len(vals) == len(ref)
        assert all(np.float32(a) == np.float32(b) for a, b in zip(vals, ref))
        assert vals == ref
