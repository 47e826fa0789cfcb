"""Python binding of libconvt, the MI355X (gfx950) ConvTranspose forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libconvt.so`` behind the C ABI declared in ``include/convt.h``.
PyTorch provides device memory and the current stream; nothing here computes
on the host, and there is no fallback: if the library is missing, importing
the functions that need it raises.

    y = convt_forward_amd.conv_transpose(x, w, bias, stride=2, padding=1)

x: [B, C_in, I...] and w: [C_in, C_out/groups, k...] are contiguous CUDA
(HIP) tensors of dtype float32, bfloat16 or float16; bias is [C_out] or None. Scalars
or per-axis tuples are accepted for stride, padding, dilation and
output_padding; padding may also give a (low, high) pair per axis, for
different padding at the two ends of an axis.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# CONVT_LIB names another build of the same library (the host-sanitizer build
# of the planner and C ABI); by default the in-tree libconvt.so is loaded
LIB_PATH = os.environ.get("CONVT_LIB") or os.path.join(_HERE, "libconvt.so")

MAX_NDIM = 3

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported request", 3: "device error"}
DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "i8": 3, "i32": 4, "i64": 5}
ROUTES = {"auto": 0, "none": 1, "fill": 2, "phase_gemm": 3, "grouped": 4, "direct": 5, "naive": 6,
          "phase_gemm_packed": 7, "phase_gemm_allphase": 8}
ROUTE_NAMES = {v: k for k, v in ROUTES.items()}
# filter layouts (element (ci, ocl, kk) of W; see include/convt.h):
#   ci_co_k [C_in][C_out/groups][k...], k_ci_co [k...][C_in][C_out/groups],
#   k_co_ci [k...][C_out][C_in/groups]
FILTER_LAYOUTS = {"ci_co_k": 0, "k_ci_co": 1, "k_co_ci": 2}
# activation applied to y after the bias (convt_activation)
ACTIVATIONS = {"none": 0, "relu": 1, "sigmoid": 2, "tanh": 3, "silu": 4, "gelu": 5}


def layout_w_shape(w_shape: Sequence[int], groups: int, layout: str) -> Tuple[int, ...]:
    """Shape of W in `layout`, from its [C_in, C_out/groups, k...] shape."""
    ci, cog, k = int(w_shape[0]), int(w_shape[1]), tuple(int(v) for v in w_shape[2:])
    if layout == "ci_co_k":
        return (ci, cog) + k
    if layout == "k_ci_co":
        return k + (ci, cog)
    if layout == "k_co_ci":
        return k + (cog * groups, ci // groups)
    raise ValueError(f"unknown filter layout {layout!r}")


def canonical_w_shape(shape: Sequence[int], groups: int, layout: str) -> Tuple[int, ...]:
    """[C_in, C_out/groups, k...] from the shape of W in `layout`."""
    shape = tuple(int(v) for v in shape)
    if layout == "ci_co_k":
        return shape
    if layout == "k_ci_co":
        return (shape[-2], shape[-1]) + shape[:-2]
    if layout == "k_co_ci":
        return (shape[-1] * groups, shape[-2] // groups) + shape[:-2]
    raise ValueError(f"unknown filter layout {layout!r}")


class ConvtError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, 'unknown status')} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("ndim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("x_shape", ctypes.c_int64 * (2 + MAX_NDIM)),
        ("w_shape", ctypes.c_int64 * (2 + MAX_NDIM)),
        ("stride", ctypes.c_int64 * MAX_NDIM),
        ("padding", ctypes.c_int64 * MAX_NDIM),
        ("dilation", ctypes.c_int64 * MAX_NDIM),
        ("output_padding", ctypes.c_int64 * MAX_NDIM),
        ("groups", ctypes.c_int64),
        ("has_bias", ctypes.c_int32),
        ("route", ctypes.c_int32),
        ("has_padding_hi", ctypes.c_int32),
        ("route_bwd", ctypes.c_int32),
        ("padding_hi", ctypes.c_int64 * MAX_NDIM),
        ("filter_layout", ctypes.c_int32),
        ("taps_flipped", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("reserved1", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("out_shape", ctypes.c_int64 * (2 + MAX_NDIM)),
        ("c_out", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("n_phases", ctypes.c_int64),
        ("useful_flops", ctypes.c_int64),
        ("route", ctypes.c_int32),
        ("route_bwd", ctypes.c_int32),
        ("bwd_workspace_bytes", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libconvt.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime; loading it first makes this library
        # bind to that same runtime (a second copy of the runtime in the
        # process, loaded by this library first, finds no device)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m convt_forward_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.convt_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(vp), ctypes.POINTER(PlanInfo)]
        L.convt_plan.restype = ctypes.c_int
        L.convt_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.convt_forward.restype = ctypes.c_int
        L.convt_prepare_weights.argtypes = [vp, vp, vp, vp]
        L.convt_prepare_weights.restype = ctypes.c_int
        L.convt_forward_prepared.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.convt_forward_prepared.restype = ctypes.c_int
        L.convt_backward_data.argtypes = [vp, vp, vp, vp, vp, vp]
        L.convt_backward_data.restype = ctypes.c_int
        L.convt_destroy.argtypes = [vp]
        L.convt_destroy.restype = None
        L.convt_status_string.argtypes = [ctypes.c_int]
        L.convt_status_string.restype = ctypes.c_char_p
        L.convt_route_name.argtypes = [ctypes.c_int32]
        L.convt_route_name.restype = ctypes.c_char_p
        p64 = ctypes.POINTER(ctypes.c_int64)
        L.convt_plan_axis_phase.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, p64, p64, p64, p64,
                                            ctypes.c_int64]
        L.convt_plan_axis_phase.restype = ctypes.c_int
        L.convt_version.argtypes = []
        L.convt_version.restype = ctypes.c_int32
        L.convt_plan_query.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.convt_plan_query.restype = ctypes.c_int
        L.convt_forward_scratch.argtypes = [vp, vp, vp, vp, vp, vp]
        L.convt_forward_scratch.restype = ctypes.c_int
        L.convt_scratch_max_bytes.argtypes = []
        L.convt_scratch_max_bytes.restype = ctypes.c_int64
        _lib = L
    return _lib


def _tup(v, nd: int, name: str) -> Tuple[int, ...]:
    if isinstance(v, int):
        return (int(v),) * nd
    v = tuple(int(t) for t in v)
    if len(v) != nd:
        raise ValueError(f"{name} must have {nd} entries")
    return v


def _pads(v, nd: int) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """(low, high) padding per axis from an int, one int per axis, or one
    (low, high) pair per axis."""
    if not isinstance(v, int) and len(v) == nd and all(not isinstance(t, int) for t in v):
        pairs = [tuple(int(u) for u in t) for t in v]
        if any(len(t) != 2 for t in pairs):
            raise ValueError("padding pairs must be (low, high)")
        return tuple(t[0] for t in pairs), tuple(t[1] for t in pairs)
    lo = _tup(v, nd, "padding")
    return lo, lo


def make_problem(x_shape: Sequence[int], w_shape: Sequence[int], stride=1, padding=0, dilation=1,
                 output_padding=0, groups: int = 1, has_bias: bool = False, dtype: str = "f32",
                 route: str = "auto", route_bwd: str = "auto", filter_layout: str = "ci_co_k",
                 taps_flipped: bool = False, activation: str = "none") -> Problem:
    """w_shape is [C_in, C_out/groups, k...] whatever filter_layout says about
    W's memory order."""
    nd = len(x_shape) - 2
    if not 1 <= nd <= MAX_NDIM or len(w_shape) != nd + 2:
        raise ValueError("x must be [B, C_in, I...] and w [C_in, C_out/groups, k...] with 1-3 spatial axes")
    p = Problem()
    p.ndim = nd
    p.dtype = DTYPES[dtype]
    for i, v in enumerate(x_shape):
        p.x_shape[i] = int(v)
    for i, v in enumerate(w_shape):
        p.w_shape[i] = int(v)
    for name in ("stride", "dilation", "output_padding"):
        arr = getattr(p, name)
        for i, v in enumerate(_tup(locals()[name], nd, name)):
            arr[i] = v
    lo, hi = _pads(padding, nd)
    for i in range(nd):
        p.padding[i] = lo[i]
        p.padding_hi[i] = hi[i]
    p.has_padding_hi = 1 if lo != hi else 0
    p.groups = int(groups)
    p.has_bias = 1 if has_bias else 0
    p.route = ROUTES[route]
    p.route_bwd = ROUTES[route_bwd]
    p.filter_layout = FILTER_LAYOUTS[filter_layout]
    p.taps_flipped = 1 if taps_flipped else 0
    p.activation = ACTIVATIONS[activation]
    return p


class Plan:
    """A validated problem (host only; building it makes no device call)."""

    def __init__(self, problem: Problem):
        self.problem = problem
        self._h = ctypes.c_void_p()
        self.info = PlanInfo()
        st = lib().convt_plan(ctypes.byref(problem), ctypes.byref(self._h), ctypes.byref(self.info))
        if st != 0:
            raise ConvtError(st, "convt_plan")
        self.ndim = problem.ndim

    @classmethod
    def create(cls, *args, **kwargs) -> "Plan":
        return cls(make_problem(*args, **kwargs))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.convt_destroy(h)
            self._h = ctypes.c_void_p()

    @property
    def handle(self) -> int:
        return self._h.value

    @property
    def out_shape(self) -> Tuple[int, ...]:
        return tuple(int(self.info.out_shape[i]) for i in range(2 + self.ndim))

    @property
    def workspace_bytes(self) -> int:
        return int(self.info.workspace_bytes)

    @property
    def route(self) -> str:
        return ROUTE_NAMES[int(self.info.route)]

    @property
    def w_layout_shape(self) -> Tuple[int, ...]:
        """The shape W has in the plan's filter layout."""
        p = self.problem
        name = {v: k for k, v in FILTER_LAYOUTS.items()}[int(p.filter_layout)]
        return layout_w_shape(tuple(p.w_shape[:2 + self.ndim]), int(p.groups), name)

    @property
    def route_bwd(self) -> str:
        return ROUTE_NAMES[int(self.info.route_bwd)]

    @property
    def bwd_workspace_bytes(self) -> int:
        return int(self.info.bwd_workspace_bytes)

    @property
    def useful_flops(self) -> int:
        return int(self.info.useful_flops)

    @property
    def n_phases(self) -> int:
        return int(self.info.n_phases)

    def axis_phase(self, axis: int, residue: int, cap: int = 64):
        """(q_count, taps, offsets) of one output residue of one spatial axis."""
        q = ctypes.c_int64()
        n = ctypes.c_int64()
        taps = (ctypes.c_int64 * cap)()
        offs = (ctypes.c_int64 * cap)()
        st = lib().convt_plan_axis_phase(self._h, axis, residue, ctypes.byref(q), ctypes.byref(n),
                                         taps, offs, cap)
        if st != 0:
            raise ConvtError(st, "convt_plan_axis_phase")
        k = min(int(n.value), cap)
        return int(q.value), [int(taps[i]) for i in range(k)], [int(offs[i]) for i in range(k)]

    # --- raw pointer entry points (integers are device addresses) ---------
    def forward_ptr(self, x: int, w: int, bias: int, y: int, workspace: int, stream: int) -> None:
        st = lib().convt_forward(self._h, x or None, w or None, bias or None, y or None,
                                 workspace or None, stream or None)
        if st != 0:
            raise ConvtError(st, "convt_forward")

    def forward_scratch_ptr(self, x: int, w: int, bias: int, y: int, stream: int) -> None:
        """convt_forward with the library's own fixed workspace (no allocation)."""
        st = lib().convt_forward_scratch(self._h, x or None, w or None, bias or None, y or None,
                                         stream or None)
        if st != 0:
            raise ConvtError(st, "convt_forward_scratch")

    def prepare_weights_ptr(self, w: int, workspace: int, stream: int) -> None:
        st = lib().convt_prepare_weights(self._h, w or None, workspace or None, stream or None)
        if st != 0:
            raise ConvtError(st, "convt_prepare_weights")

    def forward_prepared_ptr(self, x: int, w: int, bias: int, y: int, workspace: int,
                             stream: int) -> None:
        st = lib().convt_forward_prepared(self._h, x or None, w or None, bias or None, y or None,
                                          workspace or None, stream or None)
        if st != 0:
            raise ConvtError(st, "convt_forward_prepared")

    def backward_data_ptr(self, dy: int, w: int, dx: int, workspace: int, stream: int) -> None:
        st = lib().convt_backward_data(self._h, dy or None, w or None, dx or None,
                                       workspace or None, stream or None)
        if st != 0:
            raise ConvtError(st, "convt_backward_data")

    # --- torch tensors ------------------------------------------------------
    def _check(self, t, shape, name):
        import torch
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        want = self.torch_dtype
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    @property
    def torch_dtype(self):
        import torch
        return {DTYPES["f32"]: torch.float32, DTYPES["bf16"]: torch.bfloat16,
                DTYPES["f16"]: torch.float16}[int(self.problem.dtype)]

    def new_output(self, device):
        import torch
        return torch.empty(self.out_shape, dtype=self.torch_dtype, device=device)

    def new_workspace(self, device):
        import torch
        return torch.empty(max(self.workspace_bytes, 16), dtype=torch.uint8, device=device)

    def forward(self, x, w, bias=None, y=None, workspace=None, stream=None):
        """Enqueue y = convT(x, w) + bias on `stream` (default: torch's current
        stream of x's device; else a torch stream or a raw hipStream_t).
        Allocates y / the workspace with torch when not given; those
        allocations are recorded on `stream`, so the caching allocator does
        not reuse their memory before the kernels there are done. Returns y."""
        import torch
        p = self.problem
        nd = self.ndim
        self._check(x, tuple(p.x_shape[:2 + nd]), "x")
        self._check(w, self.w_layout_shape, "w")
        if p.has_bias:
            if bias is None:
                raise ValueError("the plan has a bias")
            self._check(bias, (self.out_shape[1],), "bias")
        elif bias is not None:
            raise ValueError("the plan has no bias")
        sh, ext = _launch_stream(stream, x.device)
        owned = []
        if y is None:
            y = self.new_output(x.device)
            owned.append(y)
        else:
            self._check(y, self.out_shape, "y")
        if workspace is None:
            workspace = self.new_workspace(x.device)
            owned.append(workspace)
        elif workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        self.forward_ptr(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else 0,
                         y.data_ptr(), workspace.data_ptr(), sh)
        _tie_to_stream(owned, ext)
        return y

    def new_input_grad(self, device):
        import torch
        return torch.empty(tuple(self.problem.x_shape[:2 + self.ndim]), dtype=self.torch_dtype,
                           device=device)

    def new_bwd_workspace(self, device):
        import torch
        return torch.empty(max(self.bwd_workspace_bytes, 16), dtype=torch.uint8, device=device)

    def backward_data(self, dy, w, dx=None, workspace=None, stream=None):
        """Enqueue dx = the gradient with respect to x for the upstream gradient
        dy (shape out_shape), on `stream` as in forward. Allocates dx / the
        workspace with torch when not given (recorded on `stream`). Returns
        dx."""
        import torch
        p = self.problem
        nd = self.ndim
        self._check(dy, self.out_shape, "dy")
        self._check(w, self.w_layout_shape, "w")
        sh, ext = _launch_stream(stream, dy.device)
        owned = []
        if dx is None:
            dx = self.new_input_grad(dy.device)
            owned.append(dx)
        else:
            self._check(dx, tuple(p.x_shape[:2 + nd]), "dx")
        if workspace is None:
            workspace = self.new_bwd_workspace(dy.device)
            owned.append(workspace)
        elif workspace.numel() * workspace.element_size() < self.bwd_workspace_bytes:
            raise ValueError("workspace too small")
        self.backward_data_ptr(dy.data_ptr(), w.data_ptr(), dx.data_ptr(), workspace.data_ptr(),
                               sh)
        _tie_to_stream(owned, ext)
        return dx


def _launch_stream(stream, device):
    """(raw handle, torch stream object or None) of the stream a call launches
    on: torch's current stream of `device` when `stream` is None (then None
    is returned as the object: nothing needs tying), else `stream` as given
    (a torch stream or a raw hipStream_t integer)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream, None
    if isinstance(stream, torch.cuda.Stream):
        obj = stream
    else:
        obj = torch.cuda.ExternalStream(int(stream), device=device)
    if obj.cuda_stream == torch.cuda.current_stream(device).cuda_stream:
        return obj.cuda_stream, None
    return obj.cuda_stream, obj


def _tie_to_stream(tensors, ext) -> None:
    """Tensors allocated here (on torch's current stream) but used by kernels
    enqueued on another stream: tell the caching allocator, so that their
    memory is not handed out again before that stream's work completes."""
    if ext is None:
        return
    for t in tensors:
        t.record_stream(ext)


_plan_cache: Dict[tuple, Plan] = {}


def get_plan(x_shape, w_shape, stride=1, padding=0, dilation=1, output_padding=0, groups=1,
             has_bias=False, dtype="f32", route="auto", route_bwd="auto",
             filter_layout="ci_co_k", taps_flipped=False, activation="none") -> Plan:
    """A cached plan; w_shape is [C_in, C_out/groups, k...]."""
    nd = len(x_shape) - 2
    key = (tuple(x_shape), tuple(w_shape), _tup(stride, nd, "stride"), _pads(padding, nd),
           _tup(dilation, nd, "dilation"), _tup(output_padding, nd, "output_padding"), int(groups),
           bool(has_bias), dtype, route, route_bwd, filter_layout, bool(taps_flipped), activation)
    pl = _plan_cache.get(key)
    if pl is None:
        pl = Plan.create(x_shape, w_shape, stride, padding, dilation, output_padding, groups,
                         has_bias, dtype, route, route_bwd, filter_layout, taps_flipped,
                         activation)
        _plan_cache[key] = pl
    return pl


def torch_dtype_name(t) -> str:
    import torch
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "f16"
    if t.dtype == torch.int8:
        return "i8"
    if t.dtype == torch.int32:
        return "i32"
    if t.dtype == torch.int64:
        return "i64"
    raise ValueError(f"unsupported dtype {t.dtype}")


def conv_transpose(x, w, bias=None, stride=1, padding=0, dilation=1, output_padding=0, groups=1,
                   route: str = "auto", y=None, workspace=None, stream=None,
                   filter_layout: str = "ci_co_k", taps_flipped: bool = False,
                   activation: str = "none"):
    """ConvTranspose forward on the GPU through libconvt, then `activation`
    (one of ACTIVATIONS). Returns y. w is in `filter_layout` (and spatially
    reversed when taps_flipped)."""
    pl = get_plan(tuple(x.shape), canonical_w_shape(w.shape, groups, filter_layout), stride,
                  padding, dilation, output_padding, groups, bias is not None,
                  torch_dtype_name(x), route, "auto", filter_layout, taps_flipped, activation)
    return pl.forward(x, w, bias, y=y, workspace=workspace, stream=stream)


def conv_transpose_backward_data(dy, w, x_shape, stride=1, padding=0, dilation=1,
                                 output_padding=0, groups=1, route: str = "auto", dx=None,
                                 workspace=None, stream=None, filter_layout: str = "ci_co_k",
                                 taps_flipped: bool = False):
    """Gradient of a loss with respect to the input x of conv_transpose, given
    its gradient dy with respect to the output (on the GPU through libconvt).
    Returns dx, of shape x_shape."""
    pl = get_plan(tuple(x_shape), canonical_w_shape(w.shape, groups, filter_layout), stride,
                  padding, dilation, output_padding, groups, False, torch_dtype_name(dy), "auto",
                  route, filter_layout, taps_flipped)
    return pl.backward_data(dy, w, dx=dx, workspace=workspace, stream=stream)
