"""CPU oracle for channels-last convolution forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports it, and the two share no code.

The arithmetic lives in ``oracle.cpp`` (plain direct correlation, fp64
accumulation, std::thread over output pixels); this module only marshals numpy
arrays.  See ``oracle.cpp`` for the definition and the pages it follows.

Every function here is pinned by ``tests/test_oracle_pins.py`` against brute
force, a library convolution, closed forms (1x1 = matmul, delta input) and
invariants (linearity, 3D = sum of 2D over depth taps).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_conv_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, i64p, i64p,
                                        i64p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_conv_fwd.restype = ctypes.c_int
        lib.oracle_out_shape.argtypes = [i64p] * 6
        lib.oracle_out_shape.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _triple(v, nd):
    if isinstance(v, int):
        v = (v,) * nd
    v = tuple(int(t) for t in v)
    assert len(v) == nd
    return v


def _arr(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def out_shape(in_sp, k_sp, stride, pad, dil):
    """Output spatial extents (2 or 3 dims) from the direct-convolution definition."""
    nd = len(in_sp)
    pad3 = lambda v, fill: (fill,) * (3 - nd) + tuple(v)
    out = _arr([0, 0, 0])
    rc = _lib().oracle_out_shape(_arr(pad3(in_sp, 1)), _arr(pad3(k_sp, 1)),
                                 _arr(pad3(_triple(stride, nd), 1)),
                                 _arr(pad3(_triple(pad, nd), 0)),
                                 _arr(pad3(_triple(dil, nd), 1)), out)
    if rc != 0:
        raise ValueError("invalid convolution geometry")
    return tuple(out)[3 - nd:]


def conv(x, w, stride=1, padding=0, dilation=1, rows=None, threads=0, with_den=True):
    """Direct convolution of channels-last ``x`` with ``w`` in fp64.

    x: [N,H,W,C] or [N,D,H,W,C] (any float dtype; cast to float32, which holds
    fp16/bf16 values exactly -- pass values already rounded to the GPU dtype).
    w: [O,KH,KW,C] or [O,KD,KH,KW,C].
    rows: optional int64 array of flattened output-pixel indices (n,[od,]oh,ow).
    Returns (y, den): float64 arrays [rows, O] (or the full output shape when
    rows is None); den = sum |x||w| per output.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    nd = x.ndim - 2
    assert nd in (2, 3) and w.ndim == x.ndim and w.shape[-1] == x.shape[-1]
    if nd == 2:
        n, h, wd, c = x.shape
        d = 1
        o, kh, kw, _ = w.shape
        kd = 1
    else:
        n, d, h, wd, c = x.shape
        o, kd, kh, kw, _ = w.shape
    s = _triple(stride, nd)
    p = _triple(padding, nd)
    dl = _triple(dilation, nd)
    if nd == 2:
        s, p, dl = (1,) + s, (0,) + p, (1,) + dl
    osp = out_shape((d, h, wd), (kd, kh, kw), s, p, dl)
    total = n * osp[0] * osp[1] * osp[2]
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        count = rows.size
    else:
        count = total
    y = np.empty((count, o), dtype=np.float64)
    den = np.empty((count, o), dtype=np.float64) if with_den else None
    rc = _lib().oracle_conv_fwd(
        x.ctypes.data, w.ctypes.data, _arr([n, d, h, wd, c, o, kd, kh, kw]),
        _arr(s), _arr(p), _arr(dl),
        rows.ctypes.data if rows is not None else None, count,
        y.ctypes.data, den.ctypes.data if with_den else None, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the geometry or a row index")
    if rows is None:
        shape = (n,) + (osp if nd == 3 else osp[1:]) + (o,)
        y = y.reshape(shape)
        if with_den:
            den = den.reshape(shape)
    return y, den
