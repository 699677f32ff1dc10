"""Channels-last convolution forward on AMD MI355X (gfx950) -- Python binding.

Thin ctypes marshalling over ``libcnhwc.so`` (declared in ``include/cnhwc.h``):
torch supplies device memory and the stream; every step of the convolution runs
in the library's HIP kernels.  There is no fallback: if the library is missing
this import fails, and every library error raises :class:`CnhwcError`.

    conv2d(x, w, stride, padding, dilation, *, algo, ws_limit, tile_batch, unfold_rows)
    conv3d(x, w, stride, padding, dilation, *, algo, inner_algo, ws_limit, ...)
    plan2d(...) / plan3d(...) -> Plan      (algorithm selection only; no GPU needed)

Layouts: x [N,H,W,C] / [N,D,H,W,C]; w [O,KH,KW,C] / [O,KD,KH,KW,C];
y [N,OH,OW,O] / [N,OD,OH,OW,O]; dtype float32, float16 or bfloat16 (x, w, y
share it).

``ws_limit`` is the working-set figure W the Winograd byte budget is derived
from (budget = 3/4 W - input - output - transformed filter).  It defaults to the
device's total memory, a fixed property of the device (never free memory).  For
tests, the environment variables ``CNHWC_WS_LIMIT`` (bytes) and
``CNHWC_TILE_BATCH`` are read here -- and only here -- and passed to the
library as ordinary arguments (MLX PR "Bound winograd conv2d working set by
tiling the batch", Testing: an injected budget and a forced tile size).
``CNHWC_LOG=1`` prints each call's plan to stderr.
"""
import ctypes
import functools
import os
import sys

import torch  # noqa: F401  (load torch's HIP runtime first: the library then binds to it)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcnhwc.so")

F32, F16, BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

ALGOS = {"auto": 0, "winograd": 1, "implicit_gemm": 2, "unfold_gemm": 3, "small_kd": 4,
         "winograd_half": 5}
ALGO_NAMES = {v: k for k, v in ALGOS.items()}

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "NOT_APPLICABLE", 4: "BUDGET",
          5: "WORKSPACE_TOO_SMALL", 6: "PLAN_MISMATCH", 7: "HIP", 8: "INTERNAL"}


class Desc(ctypes.Structure):
    _fields_ = [("nd", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n", ctypes.c_int64), ("d", ctypes.c_int64), ("h", ctypes.c_int64),
                ("w", ctypes.c_int64), ("c", ctypes.c_int64), ("o", ctypes.c_int64),
                ("kd", ctypes.c_int64), ("kh", ctypes.c_int64), ("kw", ctypes.c_int64),
                ("stride", ctypes.c_int32 * 3), ("pad", ctypes.c_int32 * 3),
                ("dil", ctypes.c_int32 * 3), ("groups", ctypes.c_int32)]


class Opts(ctypes.Structure):
    _fields_ = [("ws_limit_bytes", ctypes.c_uint64), ("force_algo", ctypes.c_int32),
                ("force_inner_algo", ctypes.c_int32), ("force_tile_batch", ctypes.c_int64),
                ("force_unfold_rows", ctypes.c_int64), ("force_gemm_config", ctypes.c_int32),
                ("force_split_k", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("inner_algo", ctypes.c_int32),
                ("out_d", ctypes.c_int64), ("out_h", ctypes.c_int64), ("out_w", ctypes.c_int64),
                ("tile_batch", ctypes.c_int64), ("n_tiles", ctypes.c_int64),
                ("tiles_per_image", ctypes.c_int64), ("unfold_rows", ctypes.c_int64),
                ("n_chunks", ctypes.c_int64), ("own_bytes", ctypes.c_uint64),
                ("budget_bytes", ctypes.c_uint64), ("scratch_per_element", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64), ("kernel_config", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("opts", Opts)]

    @property
    def algo_name(self):
        return ALGO_NAMES[self.algo]

    @property
    def inner_algo_name(self):
        return ALGO_NAMES[self.inner_algo]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "opts"}
        d["algo"] = self.algo_name
        d["inner_algo"] = self.inner_algo_name
        d["opts"] = {f: getattr(self.opts, f) for f, _ in Opts._fields_}
        return d

    def __repr__(self):
        return f"Plan({self.as_dict()})"


class CnhwcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: CNHWC_ERR_{self.name}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python convolution_nhwc_conv2d_amd/build.py` (needs hipcc for gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.cnhwc_abi_version.restype = ctypes.c_int
    lib.cnhwc_status_string.restype = ctypes.c_char_p
    lib.cnhwc_status_string.argtypes = [ctypes.c_int]
    lib.cnhwc_conv_select.restype = ctypes.c_int
    lib.cnhwc_conv_select.argtypes = [P(Desc), P(Opts), P(Plan)]
    lib.cnhwc_winograd_tile_rule.restype = ctypes.c_int
    lib.cnhwc_winograd_tile_rule.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             P(ctypes.c_int64), P(ctypes.c_uint64), P(ctypes.c_int32)]
    for fn in (lib.cnhwc_conv2d_fwd, lib.cnhwc_conv3d_fwd):
        fn.restype = ctypes.c_int
        fn.argtypes = [P(Desc), P(Plan), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    for fn in (lib.cnhwc_conv2d_fwd_timed, lib.cnhwc_conv3d_fwd_timed):
        fn.restype = ctypes.c_int
        fn.argtypes = [P(Desc), P(Plan), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, P(ctypes.c_void_p),
                       ctypes.c_int32, P(ctypes.c_int32)]
    lib.cnhwc_launch_count.restype = ctypes.c_int64
    lib.cnhwc_launch_count.argtypes = [P(Desc), P(Plan)]
    lib.cnhwc_conv2d_fwd_noalloc.restype = ctypes.c_int
    lib.cnhwc_conv2d_fwd_noalloc.argtypes = [P(Desc), P(Plan), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]
    if lib.cnhwc_abi_version() != 4:
        raise ImportError("libcnhwc.so ABI version mismatch")
    return lib


lib = _load()

EXPORTED = ("cnhwc_abi_version", "cnhwc_status_string", "cnhwc_conv_select",
            "cnhwc_winograd_tile_rule", "cnhwc_conv2d_fwd", "cnhwc_conv3d_fwd",
            "cnhwc_launch_count", "cnhwc_conv2d_fwd_timed", "cnhwc_conv3d_fwd_timed",
            "cnhwc_conv2d_fwd_noalloc")

# Bytes of the fixed device array cnhwc_conv2d_fwd_noalloc uses as its workspace.
NOALLOC_SCRATCH_BYTES = 64 << 20

KERNEL_KINDS = {0: "end", 1: "wino_filter", 2: "wino_input", 3: "wino_gemm", 4: "wino_output",
                5: "implicit_gemm", 6: "unfold", 7: "unfold_gemm", 8: "splitk_reduce",
                9: "wino_scale"}


# ------------------------------------------------------------------ helpers

def _tup(v, n):
    if isinstance(v, int):
        return (v,) * n
    v = tuple(int(t) for t in v)
    if len(v) != n:
        raise ValueError(f"expected {n} values, got {v}")
    return v


def make_desc(x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=torch.float32):
    """Descriptor for a 2D (4-D shapes) or 3D (5-D shapes) channels-last conv."""
    d = Desc()
    if len(x_shape) == 4:
        d.nd = 2
        n, h, w, c = x_shape
        o, kh, kw, c2 = w_shape
        dd, kd = 1, 1
        s, p, dl = (1,) + _tup(stride, 2), (0,) + _tup(padding, 2), (1,) + _tup(dilation, 2)
    elif len(x_shape) == 5:
        d.nd = 3
        n, dd, h, w, c = x_shape
        o, kd, kh, kw, c2 = w_shape
        s, p, dl = _tup(stride, 3), _tup(padding, 3), _tup(dilation, 3)
    else:
        raise ValueError("x must be 4-D (NHWC) or 5-D (NDHWC)")
    if c2 != c:
        raise ValueError(f"channel mismatch: x has {c}, w has {c2}")
    if dtype not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dtype}")
    d.dtype = _DTYPE_CODE[dtype]
    d.n, d.d, d.h, d.w, d.c, d.o, d.kd, d.kh, d.kw = n, dd, h, w, c, o, kd, kh, kw
    for i in range(3):
        d.stride[i], d.pad[i], d.dil[i] = s[i], p[i], dl[i]
    d.groups = 1
    return d


# CNHWC_LOG=1 prints each call's plan to stderr (read once, at import).
_LOG = os.environ.get("CNHWC_LOG") == "1"


@functools.lru_cache(maxsize=None)
def _total_memory(index):
    return int(torch.cuda.get_device_properties(index).total_memory)


def default_ws_limit(device=None):
    """W for the byte budget: CNHWC_WS_LIMIT if set, else the device's total
    memory (a fixed property of the device, looked up once)."""
    env = os.environ.get("CNHWC_WS_LIMIT")
    if env:
        return int(env)
    if torch.cuda.is_available():
        index = 0 if device is None else torch.device(device).index
        return _total_memory(torch.cuda.current_device() if index is None else index)
    return 288 * 10**9  # MI355X HBM3E capacity, when planning without a device


def make_opts(ws_limit=None, algo="auto", inner_algo="auto", tile_batch=None, unfold_rows=None,
              gemm_config=None, split_k=None, device=None):
    o = Opts()
    o.ws_limit_bytes = int(ws_limit) if ws_limit is not None else default_ws_limit(device)
    o.force_algo = ALGOS[algo]
    o.force_inner_algo = ALGOS[inner_algo]
    if tile_batch is None and os.environ.get("CNHWC_TILE_BATCH"):
        tile_batch = int(os.environ["CNHWC_TILE_BATCH"])
    o.force_tile_batch = int(tile_batch or 0)
    o.force_unfold_rows = int(unfold_rows or 0)
    o.force_gemm_config = int(gemm_config or 0)
    o.force_split_k = int(split_k or 0)
    return o


def select(desc, opts):
    """Run the library's planner; returns a Plan or raises CnhwcError."""
    p = Plan()
    st = lib.cnhwc_conv_select(ctypes.byref(desc), ctypes.byref(opts), ctypes.byref(p))
    if st != 0:
        raise CnhwcError(st, "cnhwc_conv_select")
    return p


def winograd_tile_rule(ws_limit, own_bytes, scratch_per_element, n, rows_per_element, force_tile=0):
    """The Winograd batch-tiling rule alone: (tile_batch, budget_bytes, fallback)."""
    t, b, f = ctypes.c_int64(), ctypes.c_uint64(), ctypes.c_int32()
    st = lib.cnhwc_winograd_tile_rule(int(ws_limit), int(own_bytes), int(scratch_per_element), int(n),
                                      int(rows_per_element), int(force_tile), ctypes.byref(t),
                                      ctypes.byref(b), ctypes.byref(f))
    if st != 0:
        raise CnhwcError(st, "cnhwc_winograd_tile_rule")
    return t.value, b.value, bool(f.value)


def plan2d(x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=torch.float32, **kw):
    return select(make_desc(x_shape, w_shape, stride, padding, dilation, dtype), make_opts(**kw))


def plan3d(x_shape, w_shape, stride=1, padding=0, dilation=1, dtype=torch.float32, **kw):
    return select(make_desc(x_shape, w_shape, stride, padding, dilation, dtype), make_opts(**kw))


def _check_tensor(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _empty_batch(x, w, stride, padding, dilation, opts, out):
    """An empty batch has an empty output and no work; the library's descriptor
    needs n >= 1, so the descriptor is checked and the output extents taken with
    n = 1, and nothing is launched."""
    desc = make_desc((1,) + tuple(x.shape[1:]), tuple(w.shape), stride, padding, dilation, x.dtype)
    plan = select(desc, opts if opts is not None else make_opts())
    oshape = (0,) + ((plan.out_d,) if desc.nd == 3 else ()) + (plan.out_h, plan.out_w, w.shape[0])
    if out is None:
        return torch.empty(oshape, dtype=x.dtype, device=x.device)
    _check_tensor(out, "out")
    if tuple(out.shape) != oshape or out.dtype != x.dtype:
        raise ValueError("out has the wrong shape or dtype")
    return out


def _run(fn, x, w, stride, padding, dilation, opts, out, workspace, plan, timer=None):
    _check_tensor(x, "x")
    _check_tensor(w, "w")
    if w.dtype != x.dtype or w.device != x.device:
        raise TypeError("x and w must share dtype and device")
    if x.shape[0] == 0:
        return _empty_batch(x, w, stride, padding, dilation,
                            opts if opts is not None or plan is None else plan.opts, out)
    desc = make_desc(tuple(x.shape), tuple(w.shape), stride, padding, dilation, x.dtype)
    if plan is None:
        plan = select(desc, opts)
    if _LOG:
        print(f"[cnhwc] x {tuple(x.shape)} w {tuple(w.shape)} {x.dtype}: {plan}", file=sys.stderr, flush=True)
    oshape = (x.shape[0],) + ((plan.out_d,) if desc.nd == 3 else ()) + (plan.out_h, plan.out_w, w.shape[0])
    if out is None:
        out = torch.empty(oshape, dtype=x.dtype, device=x.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != oshape or out.dtype != x.dtype:
            raise ValueError("out has the wrong shape or dtype")
    nbytes = int(plan.workspace_bytes)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if out.device != x.device or (workspace is not None and workspace.device != x.device):
        raise TypeError("out and workspace must be on x's device")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(x.device).cuda_stream

    def call():
        if timer is None:
            return fn(ctypes.byref(desc), ctypes.byref(plan), x.data_ptr(), w.data_ptr(), out.data_ptr(),
                      ws_ptr, ws_len, stream)
        n = lib.cnhwc_launch_count(ctypes.byref(desc), ctypes.byref(plan)) + 1
        ev, kinds = timer.slots(n)
        st_ = fn(ctypes.byref(desc), ctypes.byref(plan), x.data_ptr(), w.data_ptr(), out.data_ptr(),
                 ws_ptr, ws_len, stream, ev, n, kinds)
        if st_ == 0:
            timer.recorded(n)
        return st_

    # kernels launch on the current device, which must be the one the stream and tensors are on
    if x.device.index != torch.cuda.current_device():
        with torch.cuda.device(x.device):
            st = call()
    else:
        st = call()
    if st != 0:
        raise CnhwcError(st, fn.__name__)
    return out


class _Hip:
    """The HIP runtime torch already loaded (same SONAME), for event timing only."""
    _lib = None

    @classmethod
    def get(cls):
        if cls._lib is None:
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            cls._lib = h
        return cls._lib


class KernelTimer:
    """Per-kernel durations of forward calls, from hipEvents the library records
    on the launch stream right before each kernel (cnhwc_conv*_fwd_timed).

    Pass as ``timer=`` to conv2d/conv3d; after a synchronize, ``durations()``
    returns [(kind_name, ms), ...] for every kernel of every timed call, and
    ``call_ms`` then holds each call's span (first kernel's start event to the
    event after its last kernel), in call order."""

    def __init__(self):
        self._pending = []   # (events array, kinds array, n)
        self._pool = []
        self.call_ms = []

    def slots(self, n):
        hip = _Hip.get()
        ev = (ctypes.c_void_p * n)()
        for i in range(n):
            if self._pool:
                ev[i] = self._pool.pop()
            else:
                e = ctypes.c_void_p()
                if hip.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                ev[i] = e
        kinds = (ctypes.c_int32 * n)()
        self._cur = (ev, kinds)
        return ev, kinds

    def recorded(self, n):
        ev, kinds = self._cur
        self._pending.append((ev, kinds, n))

    def durations(self):
        hip = _Hip.get()
        out = []
        self.call_ms = []
        for ev, kinds, n in self._pending:
            hip.hipEventSynchronize(ev[n - 1])
            for i in range(n - 1):
                ms = ctypes.c_float()
                if hip.hipEventElapsedTime(ctypes.byref(ms), ev[i], ev[i + 1]) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                out.append((KERNEL_KINDS[kinds[i]], float(ms.value)))
            span = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(span), ev[0], ev[n - 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            self.call_ms.append(float(span.value))
            self._pool.extend(ev[i] for i in range(n))
        self._pending = []
        return out

    def close(self):
        hip = _Hip.get()
        for e in self._pool:
            hip.hipEventDestroy(e)
        self._pool = []


def conv2d(x, w, stride=1, padding=0, dilation=1, *, algo="auto", ws_limit=None, tile_batch=None,
           unfold_rows=None, gemm_config=None, split_k=None, out=None, workspace=None, plan=None,
           timer=None):
    """y[N,OH,OW,O] = channels-last conv2d of x[N,H,W,C] with w[O,KH,KW,C].  With
    a plan, the selection options are the plan's own and the others are unused."""
    opts = None if plan is not None else make_opts(
        ws_limit, algo, "auto", tile_batch, unfold_rows, gemm_config=gemm_config, split_k=split_k,
        device=x.device if x.is_cuda else None)
    fn = lib.cnhwc_conv2d_fwd_timed if timer is not None else lib.cnhwc_conv2d_fwd
    return _run(fn, x, w, stride, padding, dilation, opts, out, workspace, plan, timer)


def conv2d_noalloc(x, w, out, stride=1, padding=0, dilation=1, *, plan=None, algo="auto", ws_limit=None,
                   tile_batch=None, unfold_rows=None, gemm_config=None, split_k=None):
    """conv2d through cnhwc_conv2d_fwd_noalloc: the library takes the workspace
    from its fixed per-GPU device array, so nothing is allocated for the call;
    the caller passes the output ``out`` [N,OH,OW,O].  A plan whose workspace
    exceeds NOALLOC_SCRATCH_BYTES raises CnhwcError (WORKSPACE_TOO_SMALL)."""
    for t, name in ((x, "x"), (w, "w"), (out, "out")):
        _check_tensor(t, name)
    if w.dtype != x.dtype or out.dtype != x.dtype or w.device != x.device or out.device != x.device:
        raise TypeError("x, w and out must share dtype and device")
    desc = make_desc(tuple(x.shape), tuple(w.shape), stride, padding, dilation, x.dtype)
    if desc.nd != 2:
        raise ValueError("conv2d_noalloc: x must be 4-D (NHWC)")
    if plan is None:
        plan = select(desc, make_opts(ws_limit, algo, "auto", tile_batch, unfold_rows, gemm_config=gemm_config,
                                      split_k=split_k, device=x.device))
    if tuple(out.shape) != (x.shape[0], plan.out_h, plan.out_w, w.shape[0]):
        raise ValueError("out has the wrong shape")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = lib.cnhwc_conv2d_fwd_noalloc(ctypes.byref(desc), ctypes.byref(plan), x.data_ptr(), w.data_ptr(),
                                          out.data_ptr(), stream)
    if st != 0:
        raise CnhwcError(st, "cnhwc_conv2d_fwd_noalloc")
    return out


def conv3d(x, w, stride=1, padding=0, dilation=1, *, algo="auto", inner_algo="auto", ws_limit=None,
           tile_batch=None, unfold_rows=None, gemm_config=None, split_k=None, out=None, workspace=None,
           plan=None, timer=None):
    """y[N,OD,OH,OW,O] = channels-last conv3d of x[N,D,H,W,C] with w[O,KD,KH,KW,C].
    With a plan, the selection options are the plan's own and the others are unused."""
    opts = None if plan is not None else make_opts(
        ws_limit, algo, inner_algo, tile_batch, unfold_rows, gemm_config=gemm_config, split_k=split_k,
        device=x.device if x.is_cuda else None)
    fn = lib.cnhwc_conv3d_fwd_timed if timer is not None else lib.cnhwc_conv3d_fwd
    return _run(fn, x, w, stride, padding, dilation, opts, out, workspace, plan, timer)


def conv1d(x, w, stride=1, padding=0, dilation=1, **kw):
    """y[N,OL,O] = channels-last conv1d of x[N,L,C] with w[O,K,C], routed through
    the 2D path as an H = KH = 1 conv (MLX PR "Use the explicit gemm for wide
    convs on neural accelerators", Whisper follow-up: conv1d dispatches to the
    2D conv).  Keyword options as for conv2d; `out`, if given, is [N,OL,O]."""
    if x.dim() != 3 or w.dim() != 3:
        raise ValueError("conv1d: x must be [N,L,C] and w [O,K,C]")
    one = lambda v: v[0] if isinstance(v, (tuple, list)) else v
    out = kw.pop("out", None)
    y = conv2d(x.unsqueeze(1), w.unsqueeze(1), (1, one(stride)), (0, one(padding)), (1, one(dilation)),
               out=None if out is None else out.unsqueeze(1), **kw)
    return y.squeeze(1)


def direct_flops(x_shape, w_shape, plan):
    """2*N*OD*OH*OW*O*C*KD*KH*KW: the metric's flop count (direct-equivalent)."""
    o = w_shape[0]
    k = 1
    for v in w_shape[1:]:
        k *= v
    return 2 * x_shape[0] * plan.out_d * plan.out_h * plan.out_w * o * k
