"""Helpers for GPU parity tests: run the HIP path, run the oracle on the same
seeded inputs, and compare element by element.

Acceptance (per output element): |y_gpu - y| <= tol * sum|x||w|, with
tol = 2e-5 for fp32 and 1e-2 for fp16/bf16; where sum|x||w| == 0 the GPU value
must be exactly 0.
"""
import numpy as np
import torch

import oracle

TOL = {torch.float32: 2e-5, torch.float16: 1e-2, torch.bfloat16: 1e-2}


def gpu_available():
    return torch.cuda.is_available()


def to_oracle(t):
    """Exact fp32 widening of the dtype values the GPU sees."""
    return t.detach().to("cpu").float().numpy()


def check_parity(y_gpu, y_ref, den, dtype, where=""):
    """Element-wise acceptance; returns the worst |err|/den seen."""
    y = y_gpu.detach().to("cpu").double().numpy().reshape(y_ref.shape)
    tol = TOL[dtype]
    err = np.abs(y - y_ref)
    zero = den == 0
    assert np.all(np.isfinite(y)), f"{where}: non-finite output"
    assert np.all(y[zero] == 0), f"{where}: nonzero output where the window is all padding"
    bad = err > tol * den
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {int(bad.sum())} elements out of tolerance; first at {tuple(i)}: "
                             f"gpu={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} den={den[tuple(i)]!r}")
    nz = ~zero
    return float(np.max(err[nz] / den[nz])) if np.any(nz) else 0.0


def gather_rows(y_gpu, rows):
    """Rows (flattened output pixels) of a channels-last GPU output, as a CPU tensor."""
    o = y_gpu.shape[-1]
    flat = y_gpu.reshape(-1, o)
    idx = torch.as_tensor(rows, device=y_gpu.device, dtype=torch.long)
    return flat.index_select(0, idx).cpu()


def poisoned(shape, dtype, device="cuda"):
    """Output buffer prefilled with NaN so unwritten elements cannot pass."""
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def bits(t):
    """Integer view of a tensor's bits (for exact equality)."""
    t = t.detach().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t.view(torch.int16)


def tile_max(den, t):
    """Per output: the largest den among the outputs of its t x t Winograd tile
    (same image or frame, same output channel).  den is [N,(D,)OH,OW,O]."""
    d = den.reshape((-1,) + den.shape[-3:])
    out = np.empty_like(d)
    for i in range(0, d.shape[1], t):
        for j in range(0, d.shape[2], t):
            out[:, i:i + t, j:j + t] = d[:, i:i + t, j:j + t].max(axis=(1, 2), keepdims=True)
    return out.reshape(den.shape)


def check_tile_relative(y_gpu, y_ref, den, dtype, t, where=""):
    """The Winograd paths' bound: exact zero where den == 0, and
    |y_gpu - y| <= tol * (largest den among the outputs of the same t x t
    tile) elsewhere.  Returns the worst error over that tile maximum."""
    y = y_gpu.detach().to("cpu").double().numpy().reshape(y_ref.shape)
    err = np.abs(y - y_ref)
    zero = den == 0
    assert np.all(np.isfinite(y)), f"{where}: non-finite output"
    assert np.all(y[zero] == 0), f"{where}: nonzero output where every product is zero"
    tm = tile_max(den, t)
    bad = err > TOL[dtype] * tm
    assert not np.any(bad), f"{where}: {int(bad.sum())} elements beyond the tile-relative bound"
    nz = tm > 0
    return float(np.max(err[nz] / tm[nz])) if np.any(nz) else 0.0
