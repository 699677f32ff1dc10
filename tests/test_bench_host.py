"""Host logic of bench.py (no GPU): the source hash that decides whether the
stored traffic counters still apply, the counter-CSV scaling, the algorithmic
work per launch of the headline kernels, and the one-GPU guard."""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import conv_workloads as cw  # noqa: E402

cn = pytest.importorskip("convolution_nhwc_conv2d_amd")


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {  // first\n  return x + 1; /* two\n lines */ }\n"
    b = "int f(int x)\n{\n  return x + 1;\n}   // other words\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("x + 1", "x + 2"))


@pytest.fixture
def tree_copy(tmp_path, monkeypatch):
    """A copy of the sources the hash reads, with bench.ROOT pointed at it."""
    csrc = tmp_path / "convolution_nhwc_conv2d_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.HEADLINE_SOURCES:
        shutil.copy(os.path.join(ROOT, "convolution_nhwc_conv2d_amd", "csrc", f), csrc / f)
    (tmp_path / "include").mkdir()
    shutil.copy(os.path.join(ROOT, "include", "cnhwc.h"), tmp_path / "include" / "cnhwc.h")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_source_hash_follows_code_not_comments(tree_copy):
    h0 = bench.csrc_hash()
    gemm = tree_copy / "convolution_nhwc_conv2d_amd" / "csrc" / "wino_gemm.hip"
    text = gemm.read_text()
    gemm.write_text("// a new comment line\n" + text)
    assert bench.csrc_hash() == h0
    gemm.write_text(text.replace("constexpr int kResThreads = 512;", "constexpr int kResThreads = 256;"))
    assert bench.csrc_hash() != h0
    gemm.write_text(text)
    hdr = tree_copy / "include" / "cnhwc.h"
    hdr.write_text(hdr.read_text().replace("CNHWC_ALGO_WINOGRAD_HALF = 5", "CNHWC_ALGO_WINOGRAD_HALF = 6"))
    assert bench.csrc_hash() != h0


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_scales_by_the_copy_and_keys_by_hash(tree_copy):
    calib = 1 << 30
    fetch, write = tree_copy / "f.csv", tree_copy / "w.csv"
    # the copy's FETCH_SIZE reads half its bytes (KiB), WRITE_SIZE all of them
    _write_counters(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", calib / 2048),
                                          ("wino_gemm_resident_kernel<96, 6>", 1000.0),
                                          ("wino_gemm_resident_kernel<96, 6>", 3000.0),
                                          ("wino_input_kernel<float>", 500.0)])
    _write_counters(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", calib / 1024),
                                          ("wino_gemm_resident_kernel<96, 6>", 700.0),
                                          ("wino_gemm_resident_kernel<96, 6>", 700.0),
                                          ("wino_input_kernel<float>", 100.0)])
    out = bench.traffic_from(str(fetch), str(write), calib, "key")
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    # per launch: mean fetch 2000 KiB x 2 + mean write 700 KiB x 1
    assert out["kernels"]["wino_gemm"]["bytes_per_launch"] == pytest.approx((2000 * 2 + 700) * 1024)
    assert out["kernels"]["wino_input"]["bytes_per_launch"] == pytest.approx((500 * 2 + 100) * 1024)
    stored = json.load(open(tree_copy / "profiles" / "traffic.json"))
    assert stored["key"]["wino_gemm"]["csrc_hash"] == bench.csrc_hash()
    assert bench.load_traffic("key", "wino_gemm") == pytest.approx((2000 * 2 + 700) * 1024)
    # a code change voids the stored counters
    gemm = tree_copy / "convolution_nhwc_conv2d_amd" / "csrc" / "wino_gemm.hip"
    gemm.write_text(gemm.read_text() + "\nint cnhwc_unused_marker = 0;\n")
    assert bench.load_traffic("key", "wino_gemm") is None


def test_headline_work_per_launch():
    """The algorithmic work the roofline divides by, for the N=40 untiled plan:
    2*64*T*C*O flops, and the transforms' x/V and M/y bytes."""
    case = cw.wide_fp32(40)
    plan = cn.plan2d(case.x_shape(), case.w_shape(), 1, 1, 1, torch.float32, ws_limit=300 * 10**9)
    assert plan.algo_name == "winograd" and plan.n_tiles == 1 and plan.tiles_per_image == 86 * 86
    bound, flops, unit = bench.kernel_work("wino_gemm", plan, case, 4)
    assert (bound, unit) == ("mfma", "flop") and flops == 2 * 64 * 40 * 7396 * 192 * 96
    _, b_in, _ = bench.kernel_work("wino_input", plan, case, 4)
    assert b_in == 40 * 512 * 512 * 192 * 4 + 64 * 40 * 7396 * 192 * 4
    _, b_out, _ = bench.kernel_work("wino_output", plan, case, 4)
    assert b_out == 64 * 40 * 7396 * 96 * 4 + 40 * 512 * 512 * 96 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
