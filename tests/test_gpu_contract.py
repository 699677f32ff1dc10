"""GPU contract tests of the C ABI: run-to-run bit determinism of every
algorithm, errors that leave y untouched, and stream ordering with a
consumer op (MLX PR "Bound winograd conv2d working set by tiling the batch",
Problem: the failure mode there was a dropped error and a silently all-zero
output; Testing: a tiled output consumed right away)."""
import ctypes

import numpy as np
import pytest
import torch

import conv_workloads as cw
import oracle
from gpu_util import bits, check_parity, poisoned, to_oracle

pytestmark = pytest.mark.gpu

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")


def _case2(dt, c=64, o=96, n=3, h=22, w=21, seed=81):
    return cw.ConvCase(f"contract_{dt}", n, h, w, c, o, 3, 3, (1, 1), (1, 1), (1, 1), dt, "normal", "normal",
                       None, seed, c + o)


# (label, dtype, conv kind, kwargs)
RUNS = [
    ("winograd_f32", "f32", 2, dict(algo="winograd")),
    ("winograd_f32_tiled", "f32", 2, dict(algo="winograd", tile_batch=2)),
    ("implicit_f32", "f32", 2, dict(algo="implicit_gemm")),
    ("implicit_f32_split", "f32", 2, dict(algo="implicit_gemm", split_k=3)),
    ("unfold_f32", "f32", 2, dict(algo="unfold_gemm", unfold_rows=500)),
    ("implicit_f16", "f16", 2, dict(algo="implicit_gemm")),
    ("implicit_bf16_tile256", "bf16", 2, dict(algo="implicit_gemm", gemm_config=14)),
    ("unfold_bf16", "bf16", 2, dict(algo="unfold_gemm")),
    ("winograd_half_f16", "f16", 2, dict(algo="winograd_half")),
    ("winograd_half_bf16_tiled", "bf16", 2, dict(algo="winograd_half", tile_batch=2)),
    ("native3d_bf16", "bf16", 3, dict(algo="implicit_gemm")),
    ("small_kd_f16", "f16", 3, dict(algo="small_kd")),
    ("winograd_half_3d_bf16", "bf16", 3, dict(algo="winograd_half")),
]


def _inputs(dt, nd):
    if nd == 2:
        case = _case2(dt)
    else:
        case = cw.ConvCase(f"contract3d_{dt}", 1, 12, 13, 64, 48, 3, 3, (1, 1, 1), (0, 1, 1), (1, 1, 1), dt,
                           "normal", "normal", None, 82, 3, nd=3, d=6, kd=3)
    return case, case.input().cuda(), case.weight().cuda()


CANARY = 4096


@pytest.mark.parametrize("label,dt,nd,kw", RUNS, ids=[r[0] for r in RUNS])
def test_run_to_run_bits(label, dt, nd, kw):
    """Every algorithm gives the same bits on every call (fresh buffers, reused
    workspace, and after unrelated work in between), writes nothing past its
    workspace or its output (canary tails), and matches the oracle."""
    case, x, w = _inputs(dt, nd)
    fn = cn.conv2d if nd == 2 else cn.conv3d
    first = fn(x, w, **case.conv_kwargs(), **kw)
    plan = (cn.plan2d if nd == 2 else cn.plan3d)(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(),
                                                 dtype=x.dtype, **kw)
    # canaries: 4 KB of 0xA5 after the planned workspace, NaN after the output
    need = int(plan.workspace_bytes)
    ws_buf = torch.full((need + CANARY,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = ws_buf[:max(1, need)]
    numel = first.numel()
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda")  # unrelated work and allocation churn
        y_buf = poisoned((numel + CANARY,), first.dtype)
        y = fn(x, w, **case.conv_kwargs(), plan=plan, workspace=ws, out=y_buf[:numel].view(first.shape))
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(first)), f"{label}: call {rep} differs"
        assert bool((ws_buf[max(1, need):] == 0xA5).all()), f"{label}: write past the workspace"
        assert bool(torch.isnan(y_buf[numel:].float()).all()), f"{label}: write past the output"
        del junk
    yr, den = oracle.conv(to_oracle(case.input()), to_oracle(case.weight()), **case.conv_kwargs())
    check_parity(first.cpu(), yr, den, first.dtype, label)


def _st(name):
    return {v: k for k, v in cn.STATUS.items()}[name]


def _raw_call(x, w, y, ws_ptr, ws_len, plan, desc):
    stream = torch.cuda.current_stream().cuda_stream
    return cn.lib.cnhwc_conv2d_fwd(ctypes.byref(desc), ctypes.byref(plan), x.data_ptr(), w.data_ptr(),
                                   y.data_ptr(), ws_ptr, ws_len, stream)


@pytest.mark.parametrize("algo", ["winograd", "winograd_half", "unfold_gemm", "implicit_gemm"])
def test_errors_leave_y_untouched(algo):
    """A call that fails validation queues nothing: y keeps its NaN fill."""
    dt = "f16" if algo == "winograd_half" else "f32"
    case = _case2(dt)
    x, w = case.input().cuda(), case.weight().cuda()
    kw = dict(algo=algo, split_k=3) if algo == "implicit_gemm" else dict(algo=algo)
    plan = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, x.dtype, **kw)
    desc = cn.make_desc(tuple(x.shape), tuple(w.shape), 1, 1, 1, x.dtype)
    y = poisoned((case.n, case.h, case.w, case.o), x.dtype)
    need = int(plan.workspace_bytes)
    assert need > 0
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    # workspace one byte too small
    st = _raw_call(x, w, y, ws.data_ptr(), need - 1, plan, desc)
    assert st == _st("WORKSPACE_TOO_SMALL")
    # misaligned workspace and output pointers
    assert _raw_call(x, w, y, ws.data_ptr() + 8, need, plan, desc) == _st("INVALID_ARGUMENT")
    y_off = poisoned((case.n * case.h * case.w * case.o + 8,), x.dtype)
    stream = torch.cuda.current_stream().cuda_stream
    st = cn.lib.cnhwc_conv2d_fwd(ctypes.byref(desc), ctypes.byref(plan), x.data_ptr(), w.data_ptr(),
                                 y_off.data_ptr() + 2, ws.data_ptr(), need, stream)
    assert st == _st("INVALID_ARGUMENT")
    # a plan that does not match the descriptor
    other = cn.make_desc((case.n, case.h + 1, case.w, case.c), tuple(w.shape), 1, 1, 1, x.dtype)
    st = cn.lib.cnhwc_conv2d_fwd(ctypes.byref(other), ctypes.byref(plan), x.data_ptr(), w.data_ptr(),
                                 y.data_ptr(), ws.data_ptr(), need, stream)
    assert st == _st("PLAN_MISMATCH")
    # the workspace overlapping y
    assert _raw_call(x, w, y, y.data_ptr(), need, plan, desc) == _st("INVALID_ARGUMENT")
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all() and torch.isnan(y_off.float()).all()
    # and the same call with a valid workspace writes every element
    assert _raw_call(x, w, y, ws.data_ptr(), need, plan, desc) == 0
    torch.cuda.synchronize()
    assert not torch.isnan(y.float()).any()


def test_consumer_on_the_same_stream_sees_the_tiled_output():
    """A torch op queued right after the call, with no synchronisation, reads
    the finished tiled Winograd output (stream order is the only guarantee)."""
    case = cw.ConvCase("contract_consumer", 6, 40, 44, 64, 96, 3, 3, (1, 1), (1, 1), (1, 1), "f32", "uniform",
                       "normal", None, 83, 0)
    x, w = case.input().cuda(), case.weight().cuda()
    y = cn.conv2d(x, w, 1, 1, 1, algo="winograd", tile_batch=2, out=poisoned((6, 40, 44, 96), torch.float32))
    s = y.double().sum(dim=(1, 2, 3))  # consumer, same stream, no sync in between
    ref = cn.conv2d(x, w, 1, 1, 1, algo="winograd")
    torch.cuda.synchronize()
    assert torch.equal(s, ref.double().sum(dim=(1, 2, 3)))
    assert np.isfinite(s.cpu().numpy()).all()


def test_empty_batch_returns_an_empty_output():
    """N = 0: the binding returns an empty output of the planned shape and
    launches nothing (the C descriptor needs n >= 1); the rest of the
    descriptor is still checked."""
    for dt in (torch.float32, torch.bfloat16):
        x = torch.empty((0, 12, 10, 32), dtype=dt, device="cuda")
        w = torch.zeros((48, 3, 3, 32), dtype=dt, device="cuda")
        y = cn.conv2d(x, w, 2, 1, 1)
        assert y.shape == (0, 6, 5, 48) and y.dtype == dt
        out = torch.empty((0, 6, 5, 48), dtype=dt, device="cuda")
        assert cn.conv2d(x, w, 2, 1, 1, out=out) is out
        with pytest.raises(ValueError):
            cn.conv2d(x, w, 1, 1, 1, out=out)
        with pytest.raises(cn.CnhwcError) as e:
            cn.conv2d(x, w, 0, 1, 1)
        assert e.value.name == "INVALID_ARGUMENT"
    x3 = torch.empty((0, 5, 8, 8, 16), dtype=torch.bfloat16, device="cuda")
    w3 = torch.zeros((16, 3, 3, 3, 16), dtype=torch.bfloat16, device="cuda")
    assert cn.conv3d(x3, w3, 1, (0, 1, 1), 1).shape == (0, 3, 8, 8, 16)
    x1 = torch.empty((0, 50, 16), dtype=torch.float16, device="cuda")
    w1 = torch.zeros((24, 3, 16), dtype=torch.float16, device="cuda")
    assert cn.conv1d(x1, w1, 1, 1).shape == (0, 50, 24)


@pytest.mark.parametrize("algo,dt", [("winograd", "f32"), ("winograd_half", "bf16"), ("implicit_gemm", "f16")])
def test_concurrent_calls_on_two_streams(algo, dt):
    """The library keeps no mutable state of its own (scales, partial maxima
    and transformed operands live in the caller's workspace), so calls queued
    on two streams at once give the bits each gives alone."""
    cases = [_case2(dt, seed=90 + i) for i in range(2)]
    xs = [c.input().cuda() for c in cases]
    ws_ = [c.weight().cuda() for c in cases]
    alone = [cn.conv2d(x, w, 1, 1, 1, algo=algo) for x, w in zip(xs, ws_)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ys = [None, None]
    ev = torch.cuda.Event()
    ev.record()
    for i in range(2):
        streams[i].wait_event(ev)
        with torch.cuda.stream(streams[i]):
            ys[i] = cn.conv2d(xs[i], ws_[i], 1, 1, 1, algo=algo)
    torch.cuda.synchronize()
    for y, a in zip(ys, alone):
        assert torch.equal(bits(y), bits(a))
