"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module is shared by the tests, the benchmark and the smoke check.  It holds
no convolution arithmetic: only shapes and random draws.  Both the oracle and the
HIP path receive the tensors it returns.

Draws use numpy's PCG64 (``default_rng([seed, case, kind, index])``) in float32
and are then rounded to the target dtype with round-to-nearest-even (torch
``.to()``).  Each batch element (or frame) has its own stream, so any subset of
elements can be regenerated on its own.

Value distributions follow the workloads the MLX pages measure:
  * fp32 2D convs (the Winograd tiling page, its reported 512x512, 192->96 fp32
    shape): x ~ U[-1, 1], w ~ N(0, 1/(9C));
  * half-precision sweeps and the ResNet-50 stack (the explicit-gemm page, its
    C_out table, K axis, Verified grid and ResNet-50 tables): x ~ N(0,1),
    w ~ N(0, 1/K) with K = KH*KW*C;
  * 3D (the small-kernel-depth page, its bf16 3x3x3 timing table):
    x ~ N(0,1), w ~ N(0, 1/(27C)).
No dataset is involved: the ResNet-50 stack is only a list of conv shapes.
"""
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

_KIND_W, _KIND_X = 0, 1


def _rng(seed: int, case: int, kind: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(case), int(kind), int(index)])


def _draw(g: np.random.Generator, dist: str, shape, scale: float) -> np.ndarray:
    if dist == "uniform":
        return (g.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)) * np.float32(scale)
    if dist == "normal":
        return g.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    if dist == "ternary":  # integers in {-1, 0, 1}: every partial sum stays exact
        return g.integers(-1, 2, size=shape).astype(np.float32)
    raise ValueError(dist)


@dataclass
class ConvCase:
    """One convolution workload (2D when d == kd == 1 and nd == 2)."""
    name: str
    n: int
    h: int
    w: int
    c: int
    o: int
    kh: int
    kw: int
    stride: Tuple[int, ...] = (1, 1)
    pad: Tuple[int, ...] = (0, 0)
    dil: Tuple[int, ...] = (1, 1)
    dtype: str = "f32"
    x_dist: str = "uniform"     # "uniform" (U[-1,1]), "normal" (N(0,1)), "ternary"
    w_dist: str = "normal"
    w_std: Optional[float] = None  # default 1/sqrt(KH*KW*C[*KD]) (i.e. var 1/K)
    seed: int = 1
    case: int = 0
    nd: int = 2
    d: int = 1
    kd: int = 1

    @property
    def K(self) -> int:
        return self.kd * self.kh * self.kw * self.c

    def x_shape(self, n=None):
        n = self.n if n is None else n
        return (n, self.h, self.w, self.c) if self.nd == 2 else (n, self.d, self.h, self.w, self.c)

    def w_shape(self):
        return (self.o, self.kh, self.kw, self.c) if self.nd == 2 else (self.o, self.kd, self.kh, self.kw, self.c)

    def weight(self) -> torch.Tensor:
        std = self.w_std if self.w_std is not None else 1.0 / math.sqrt(self.K)
        a = _draw(_rng(self.seed, self.case, _KIND_W, 0), self.w_dist, self.w_shape(), std)
        return torch.from_numpy(a).to(DTYPES[self.dtype])

    def element(self, i: int) -> torch.Tensor:
        """Batch element i (shape x_shape()[1:]), from its own stream."""
        a = _draw(_rng(self.seed, self.case, _KIND_X, i), self.x_dist, self.x_shape(1)[1:], 1.0)
        return torch.from_numpy(a).to(DTYPES[self.dtype])

    def input(self, elements: Optional[Sequence[int]] = None) -> torch.Tensor:
        """Input for all batch elements (or the listed ones), stacked."""
        idx = range(self.n) if elements is None else elements
        out = torch.empty((len(idx),) + self.x_shape(1)[1:], dtype=DTYPES[self.dtype])
        for j, i in enumerate(idx):
            out[j] = self.element(i)
        return out

    def conv_kwargs(self):
        return dict(stride=tuple(self.stride), padding=tuple(self.pad), dilation=tuple(self.dil))


# ---------------------------------------------------------------- workloads

def small_fp32(seed: int = 1) -> ConvCase:
    """N=1, 16x16, 32->32, 3x3, stride 1, pad 1, fp32; x ~ U[-1,1], w ~ N(0, 1/(9C))."""
    return ConvCase("small_fp32_16x16_32to32", 1, 16, 16, 32, 32, 3, 3, (1, 1), (1, 1), (1, 1),
                    "f32", "uniform", "normal", 1.0 / math.sqrt(9 * 32), seed, 0)


def wide_fp32(n: int, h: int = 512, w: int = 512, c: int = 192, o: int = 96, seed: int = 2) -> ConvCase:
    """The fp32 Winograd-tiling workload: n x 512x512, 192->96, 3x3, s1, p1."""
    # the case index does not depend on n: element i is the same for every batch size
    return ConvCase(f"fp32_{n}x{h}x{w}_{c}to{o}", n, h, w, c, o, 3, 3, (1, 1), (1, 1), (1, 1),
                    "f32", "uniform", "normal", 1.0 / math.sqrt(9 * c), seed, 0)


def half_geometry_grid(dtype: str, c_in: int, seed: int = 3) -> List[ConvCase]:
    """Filter {3,5,7} x stride {1,2} x dilation {1,2} x pad {0,1,2}, plus 1x1 cases,
    C_out = 128, N = 1, input sized so OH = OW = 16 (or the largest fitting)."""
    cases = []
    idx = 0
    for k in (1, 3, 5, 7):
        for s in (1, 2):
            for dl in ((1, 2) if k > 1 else (1,)):
                for p in (0, 1, 2):
                    # choose H so that OH = 16 exactly: H = (16-1)*s + dl*(k-1) + 1 - 2p
                    h = (16 - 1) * s + dl * (k - 1) + 1 - 2 * p
                    cases.append(ConvCase(f"grid_{dtype}_k{k}s{s}d{dl}p{p}_c{c_in}", 1, h, h, c_in, 128,
                                          k, k, (s, s), (p, p), (dl, dl), dtype, "normal", "normal",
                                          None, seed, 1000 * c_in + idx))
                    idx += 1
    return cases


def cout_axis(dtype: str, c_out: int, n: int, c_in: int = 256, seed: int = 3) -> ConvCase:
    """3x3 s1 d1 p1 on 32x32, C_in=256, C_out in {128..4096}, M = n*1024."""
    return ConvCase(f"cout_{dtype}_n{n}_c{c_in}_o{c_out}", n, 32, 32, c_in, c_out, 3, 3, (1, 1), (1, 1),
                    (1, 1), dtype, "normal", "normal", None, seed, 10 * c_out + n + c_in)


RESNET50_LAYERS = [
    # (spatial_in, C, O, k, stride, multiplicity, stage)
    (224, 3, 64, 7, 2, 1, "stem"),
    (56, 64, 64, 1, 1, 1, "layer1"), (56, 64, 64, 3, 1, 3, "layer1"), (56, 64, 256, 1, 1, 4, "layer1"),
    (56, 256, 64, 1, 1, 2, "layer1"),
    (56, 256, 128, 1, 1, 1, "layer2"), (56, 128, 128, 3, 2, 1, "layer2"), (56, 256, 512, 1, 2, 1, "layer2"),
    (28, 128, 512, 1, 1, 4, "layer2"), (28, 128, 128, 3, 1, 3, "layer2"), (28, 512, 128, 1, 1, 3, "layer2"),
    (28, 512, 256, 1, 1, 1, "layer3"), (28, 256, 256, 3, 2, 1, "layer3"), (28, 512, 1024, 1, 2, 1, "layer3"),
    (14, 256, 1024, 1, 1, 6, "layer3"), (14, 256, 256, 3, 1, 5, "layer3"), (14, 1024, 256, 1, 1, 5, "layer3"),
    (14, 1024, 512, 1, 1, 1, "layer4"), (14, 512, 512, 3, 2, 1, "layer4"), (14, 1024, 2048, 1, 2, 1, "layer4"),
    (7, 512, 2048, 1, 1, 3, "layer4"), (7, 512, 512, 3, 1, 2, "layer4"), (7, 2048, 512, 1, 1, 2, "layer4"),
]


def resnet50_layers(batch: int, dtype: str = "f16", seed: int = 4) -> List[Tuple[ConvCase, int, str]]:
    """The ResNet-50 (v1.5) conv shapes: (case, multiplicity, stage)."""
    out = []
    for i, (sp, c, o, k, s, mult, stage) in enumerate(RESNET50_LAYERS):
        p = k // 2
        out.append((ConvCase(f"resnet50_{stage}_{i}_{sp}_{c}to{o}_k{k}s{s}", batch, sp, sp, c, o, k, k,
                             (s, s), (p, p), (1, 1), dtype, "normal", "normal", None, seed, 100 * batch + i),
                    mult, stage))
    return out


def video3d(t: int, h: int, w: int, c: int, o: int, dtype: str = "bf16", seed: int = 5) -> ConvCase:
    """conv3d N=1, 3x3x3, stride 1, pad (0,1,1); x ~ N(0,1), w ~ N(0, 1/(27C))."""
    return ConvCase(f"conv3d_{dtype}_{t}x{h}x{w}_{c}to{o}", 1, h, w, c, o, 3, 3, (1, 1, 1), (0, 1, 1),
                    (1, 1, 1), dtype, "normal", "normal", 1.0 / math.sqrt(27 * c), seed, t * 100000 + h + c,
                    nd=3, d=t, kd=3)


VIDEO3D_SHAPES = [(17, 64, 64, 256, 256), (41, 60, 104, 256, 256), (41, 120, 208, 512, 512)]


def sample_rows(total: int, count: int, seed: int) -> np.ndarray:
    """Seeded, sorted, distinct output-row indices (for oracle subsets)."""
    count = min(count, total)
    g = np.random.default_rng([int(seed), 777])
    return np.sort(g.choice(total, size=count, replace=False)).astype(np.int64)
