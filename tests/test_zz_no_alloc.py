"""GPU tests of the allocation-free entry point cnhwc_conv2d_fwd_noalloc: its
output equals cnhwc_conv2d_fwd's (same plan, caller-allocated workspace) bit
for bit, and the oracle's within the tolerance, on two calls in a row, the
second smaller than the first (the fixed scratch array then holds the first
call's contents).  Plans whose workspace exceeds the array are rejected
before any work is queued.
"""
import numpy as np
import pytest
import torch

import conv_workloads as cw
import oracle
from gpu_util import bits, check_parity, poisoned, to_oracle

pytestmark = pytest.mark.gpu

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")


def _case(name, n, h, w, c, o, dtype, seed, k=3, p=1):
    return cw.ConvCase(name, n, h, w, c, o, k, k, (1, 1), (p, p), (1, 1), dtype, "uniform" if dtype == "f32" else
                       "normal", "normal", None, seed, 0)


# (algo, extra options, first case, second (smaller) case)
SEQUENCES = [
    ("winograd", {}, _case("wino_a", 3, 40, 44, 64, 64, "f32", 31), _case("wino_b", 1, 20, 18, 32, 48, "f32", 32)),
    ("winograd_half", {}, _case("wh_a", 2, 32, 36, 64, 64, "f16", 33), _case("wh_b", 1, 16, 12, 32, 32, "f16", 34)),
    ("winograd_half", {}, _case("whb_a", 2, 30, 32, 96, 64, "bf16", 35),
     _case("whb_b", 1, 9, 14, 32, 16, "bf16", 36)),
    ("implicit_gemm", {"split_k": 4}, _case("sk_a", 1, 8, 8, 256, 96, "f16", 37),
     _case("sk_b", 1, 4, 6, 128, 40, "f16", 38)),
    ("unfold_gemm", {"unfold_rows": 100}, _case("uf_a", 2, 17, 19, 24, 40, "bf16", 39),
     _case("uf_b", 1, 7, 9, 16, 24, "bf16", 40)),
    ("implicit_gemm", {}, _case("ig_a", 2, 16, 16, 64, 64, "f32", 41), _case("ig_b", 1, 8, 8, 32, 32, "f32", 42)),
]


def _plan(case, algo, extra):
    return cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs(), dtype=cw.DTYPES[case.dtype], algo=algo,
                     **extra)


@pytest.mark.parametrize("seq", SEQUENCES, ids=[f"{s[0]}_{s[2].name}" for s in SEQUENCES])
def test_noalloc_matches_workspace_entry_point(seq):
    algo, extra, first, second = seq
    for case in (first, second):
        plan = _plan(case, algo, extra)
        assert plan.algo_name == algo
        assert plan.workspace_bytes <= cn.NOALLOC_SCRATCH_BYTES
        if algo != "implicit_gemm" or extra:
            assert plan.workspace_bytes > 0, "the sequence must exercise the scratch array"
        x, w = case.input(), case.weight()
        xg, wg = x.to("cuda"), w.to("cuda")
        oshape = (x.shape[0], plan.out_h, plan.out_w, w.shape[0])
        y_na = cn.conv2d_noalloc(xg, wg, poisoned(oshape, x.dtype), **case.conv_kwargs(), plan=plan)
        y_ws = cn.conv2d(xg, wg, **case.conv_kwargs(), plan=plan, out=poisoned(oshape, x.dtype))
        torch.cuda.synchronize()
        assert torch.equal(bits(y_na), bits(y_ws)), f"{case.name}: noalloc bits differ from the workspace call"
        yr, den = oracle.conv(to_oracle(x), to_oracle(w), **case.conv_kwargs())
        check_parity(y_na.cpu(), yr, den, y_na.dtype, f"{case.name}/{algo}/noalloc")


def test_noalloc_repeated_calls_give_the_same_bits():
    """Back-to-back calls on one stream: the second call reads nothing the first left behind."""
    case = SEQUENCES[0][2]
    plan = _plan(case, "winograd", {})
    x, w = case.input().to("cuda"), case.weight().to("cuda")
    oshape = (x.shape[0], plan.out_h, plan.out_w, w.shape[0])
    ys = [cn.conv2d_noalloc(x, w, poisoned(oshape, x.dtype), **case.conv_kwargs(), plan=plan) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(bits(y), bits(ys[0]))


def test_noalloc_rejects_a_plan_over_the_array():
    """A Winograd plan whose scratch exceeds the fixed array: WORKSPACE_TOO_SMALL,
    nothing queued, y untouched."""
    case = _case("big", 8, 128, 128, 64, 64, "f32", 43)
    plan = _plan(case, "winograd", {})
    assert plan.workspace_bytes > cn.NOALLOC_SCRATCH_BYTES
    x, w = case.input().to("cuda"), case.weight().to("cuda")
    y = poisoned((8, plan.out_h, plan.out_w, 64), torch.float32)
    with pytest.raises(cn.CnhwcError) as e:
        cn.conv2d_noalloc(x, w, y, **case.conv_kwargs(), plan=plan)
    assert e.value.name == "WORKSPACE_TOO_SMALL"
    torch.cuda.synchronize()
    assert bool(torch.isnan(y).all())
