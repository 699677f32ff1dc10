"""The C-ABI library loads, exports every function include/cnhwc.h declares, and
rejects bad calls before queueing any work (no GPU needed: every call here
returns during validation, so the placeholder pointers are never touched).
"""
import ctypes
import os
import re

import pytest
import torch

import convolution_nhwc_conv2d_amd as cn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cnhwc.h")


def test_every_declared_function_is_exported():
    text = re.sub(r"/\*.*?\*/", " ", open(HEADER).read(), flags=re.S)  # drop comments
    names = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(cnhwc_\w+)\s*\(", text, re.M))
    assert names == set(cn.EXPORTED)
    for n in names:
        assert hasattr(cn.lib, n), n


def test_header_constants_match_binding_layout():
    text = open(HEADER).read()
    assert int(re.search(r"#define CNHWC_ABI_VERSION (\d+)", text).group(1)) == cn.lib.cnhwc_abi_version()
    # struct sizes as a C compiler lays them out
    assert ctypes.sizeof(cn.Desc) == 4 + 4 + 9 * 8 + 3 * 12 + 4
    assert ctypes.sizeof(cn.Opts) == 8 + 4 + 4 + 8 + 8 + 4 + 4


def test_single_hip_runtime_in_process():
    maps = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
    assert len(set(maps)) <= 1, set(maps)


def test_status_strings():
    for code in range(9):
        assert cn.lib.cnhwc_status_string(code)
    assert cn.lib.cnhwc_status_string(0) == b"ok"


# fake but 256-byte-aligned device addresses: validation never dereferences them
X, W, Y, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _call(fn, desc, plan, x=X, w=W, y=Y, ws=WS, nbytes=None):
    if nbytes is None:
        nbytes = plan.workspace_bytes
    return fn(ctypes.byref(desc), ctypes.byref(plan), x, w, y, ws, nbytes, None)


def _wino():
    d = cn.make_desc((2, 64, 64, 64), (96, 3, 3, 64), 1, 1, 1, torch.float32)
    p = cn.select(d, cn.make_opts(ws_limit=10**12, algo="winograd"))
    return d, p


def test_workspace_too_small():
    d, p = _wino()
    assert p.workspace_bytes > 0
    assert _call(cn.lib.cnhwc_conv2d_fwd, d, p, nbytes=p.workspace_bytes - 1) == 5


def test_null_and_misaligned_pointers():
    d, p = _wino()
    f = cn.lib.cnhwc_conv2d_fwd
    assert _call(f, d, p, x=None) == 1
    assert _call(f, d, p, y=Y + 4) == 1
    assert _call(f, d, p, ws=None) == 1
    assert _call(f, d, p, y=X) == 1  # y overlaps x


def test_overlapping_buffers():
    """y and the workspace may overlap nothing; x and w may share memory."""
    d, p = _wino()
    f = cn.lib.cnhwc_conv2d_fwd
    wb = 96 * 9 * 64 * 4
    assert _call(f, d, p, y=W + wb - 256) == 1     # y starts inside w
    assert _call(f, d, p, ws=W + 256) == 1         # workspace inside w
    assert _call(f, d, p, ws=Y + 256) == 1         # workspace inside y
    assert _call(f, d, p, ws=X) == 1               # workspace on x


def test_plan_mismatch():
    d, p = _wino()
    p.tile_batch = 1
    assert _call(cn.lib.cnhwc_conv2d_fwd, d, p) == 6
    d, p = _wino()
    d.n = 3
    assert _call(cn.lib.cnhwc_conv2d_fwd, d, p) == 6


def test_wrong_entry_point_for_rank():
    d, p = _wino()
    assert _call(cn.lib.cnhwc_conv3d_fwd, d, p) == 1
    d3 = cn.make_desc((1, 5, 8, 8, 32), (32, 3, 3, 3, 32), 1, (0, 1, 1), 1, torch.bfloat16)
    p3 = cn.select(d3, cn.make_opts())
    assert _call(cn.lib.cnhwc_conv2d_fwd, d3, p3) == 1


def test_select_null_arguments():
    d = cn.make_desc((1, 8, 8, 8), (8, 3, 3, 8), 1, 1, 1)
    assert cn.lib.cnhwc_conv_select(None, ctypes.byref(cn.make_opts()), ctypes.byref(cn.Plan())) == 1
    assert cn.lib.cnhwc_conv_select(ctypes.byref(d), None, ctypes.byref(cn.Plan())) == 1


def test_tile_rule_arguments():
    with pytest.raises(cn.CnhwcError):
        cn.winograd_tile_rule(10**9, 0, 0, 1, 1)  # zero scratch
    assert cn.winograd_tile_rule(2**64 - 1, 0, 1, 5, 1) == (5, (2**64 - 1) // 4 * 3 + 2, False)
