"""CPU oracle for the ConvTranspose forward pass and its input gradient
(double precision).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only code that may import this package. The GPU library
and its Python binding never import it, and the two share no code.

The arithmetic lives in ``convt_oracle.c`` (plain C, double precision, a
scatter-add written out from the definition; see that file's header for the
passages it follows). This module compiles it with gcc and calls it through
ctypes. Every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` against closed forms, library routines, hand
computed cases and identities that the pages state; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convt_oracle.c")
_LIB = os.path.join(_HERE, "libconvt_oracle.so")


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle library with gcc (-O3 -fopenmp). Returns its path."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    p64 = ctypes.POINTER(ctypes.c_int64)
    pd = ctypes.POINTER(ctypes.c_double)
    # (ndim, x_shape, w_shape, stride, padding, padding_end, dilation, output_padding, groups, ...)
    lib.convt_oracle_out_shape.argtypes = [ctypes.c_int, p64, p64, p64, p64, p64, p64, p64,
                                           ctypes.c_int64, p64]
    lib.convt_oracle_out_shape.restype = ctypes.c_int
    lib.convt_oracle_forward.argtypes = [ctypes.c_int, p64, p64, p64, p64, p64, p64, p64,
                                         ctypes.c_int64, pd, pd, pd, pd, pd, ctypes.c_int]
    lib.convt_oracle_forward.restype = ctypes.c_int
    lib.convt_oracle_points.argtypes = [ctypes.c_int, p64, p64, p64, p64, p64, p64, p64,
                                        ctypes.c_int64, pd, pd, pd, ctypes.c_int64, p64, pd,
                                        pd, ctypes.c_int]
    lib.convt_oracle_points.restype = ctypes.c_int
    lib.convt_oracle_activation.argtypes = [ctypes.c_int, pd, pd, ctypes.c_int64]
    lib.convt_oracle_activation.restype = ctypes.c_int
    lib.convt_oracle_backward_data.argtypes = [ctypes.c_int, p64, p64, p64, p64, p64, p64, p64,
                                               ctypes.c_int64, pd, pd, pd, pd, ctypes.c_int]
    lib.convt_oracle_backward_data.restype = ctypes.c_int
    lib.convt_oracle_backward_data_points.argtypes = [ctypes.c_int, p64, p64, p64, p64, p64, p64,
                                                      p64, ctypes.c_int64, pd, pd, ctypes.c_int64,
                                                      p64, pd, pd, ctypes.c_int]
    lib.convt_oracle_backward_data_points.restype = ctypes.c_int
    lib.convt_oracle_max_threads.argtypes = []
    lib.convt_oracle_max_threads.restype = ctypes.c_int
    return lib


def _i64(v: Sequence[int]):
    a = np.ascontiguousarray(np.asarray(v, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _f64(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _attrs(x_shape, w_shape, stride, padding, dilation, output_padding):
    """(ndim, stride, low padding, high padding, dilation, output_padding) per axis.

    padding: an int, one int per axis (both ends), or one (low, high) pair per
    axis (the AWS Neuron conv3d_transpose page's asymmetric form)."""
    nd = len(x_shape) - 2
    if len(w_shape) != nd + 2:
        raise ValueError("x and W ranks differ")

    def tup(v, default):
        if v is None:
            return (default,) * nd
        if isinstance(v, int):
            return (v,) * nd
        if len(v) != nd:
            raise ValueError("attribute rank mismatch")
        return tuple(int(t) for t in v)

    if padding is not None and not isinstance(padding, int) and len(padding) == nd and \
            all(not isinstance(v, (int, np.integer)) for v in padding):
        lo = tuple(int(v[0]) for v in padding)
        hi = tuple(int(v[1]) for v in padding)
    else:
        lo = hi = tup(padding, 0)
    return (nd, tup(stride, 1), lo, hi, tup(dilation, 1), tup(output_padding, 0))


class Oracle:
    """The oracle library behind one compiled build of ``convt_oracle.c``."""

    def __init__(self, path: str):
        self.path = path
        self.lib = _bind(path)

    def max_threads(self) -> int:
        return int(self.lib.convt_oracle_max_threads())

    def out_shape(self, x_shape, w_shape, stride=None, padding=None, dilation=None,
                  output_padding=None, groups: int = 1) -> Tuple[int, ...]:
        """Output shape [B, C_out, O...]; raises ValueError for an ill-formed problem."""
        nd, s, p, ph, d, op = _attrs(x_shape, w_shape, stride, padding, dilation, output_padding)
        keep = [_i64(x_shape), _i64(w_shape), _i64(s), _i64(p), _i64(ph), _i64(d), _i64(op)]
        out = np.zeros(2 + nd, dtype=np.int64)
        rc = self.lib.convt_oracle_out_shape(nd, *[k[1] for k in keep], int(groups),
                                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        if rc != 0:
            raise ValueError("ill-formed transposed convolution")
        return tuple(int(v) for v in out)

    def activation(self, act: int, v: np.ndarray) -> np.ndarray:
        """The activation with code act (0 none, 1 ReLU, 2 sigmoid, 3 tanh,
        4 SiLU, 5 GELU) applied to each element of v, in float64."""
        a = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty_like(a)
        rc = self.lib.convt_oracle_activation(int(act), a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                              int(a.size))
        if rc != 0:
            raise ValueError(f"unknown activation {act}")
        return out

    def forward(self, x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray] = None,
                stride=None, padding=None, dilation=None, output_padding=None, groups: int = 1,
                with_scale: bool = True, nthreads: int = 0, activation: int = 0):
        """Full forward pass in float64, then the activation (code as in
        activation()). Returns (y, scale); scale (the magnitude sum of the
        terms before the activation) is None unless asked."""
        nd, s, p, ph, d, op = _attrs(x.shape, w.shape, stride, padding, dilation, output_padding)
        oshape = self.out_shape(x.shape, w.shape, s, list(zip(p, ph)), d, op, groups)
        xa, xp = _f64(x)
        wa, wp = _f64(w)
        ba, bp = _f64(bias)
        if ba is not None and ba.shape != (oshape[1],):
            raise ValueError("bias must have shape [C_out]")
        y = np.empty(oshape, dtype=np.float64)
        sc = np.empty(oshape, dtype=np.float64) if with_scale else None
        keep = [_i64(x.shape), _i64(w.shape), _i64(s), _i64(p), _i64(ph), _i64(d), _i64(op)]
        rc = self.lib.convt_oracle_forward(
            nd, *[k[1] for k in keep], int(groups), xp, wp, bp,
            y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            sc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if sc is not None else None,
            int(nthreads))
        if rc != 0:
            raise ValueError("ill-formed transposed convolution")
        if activation:
            y = self.activation(activation, y)
        return y, sc

    def points(self, x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], pts: np.ndarray,
               stride=None, padding=None, dilation=None, output_padding=None, groups: int = 1,
               nthreads: int = 0, activation: int = 0):
        """Outputs at the given points, each computed on its own, then the
        activation.

        ``pts`` is an int array [n, 2 + ndim] of (b, oc, o...). Returns (y, scale)
        as float64 arrays of length n.
        """
        nd, s, p, ph, d, op = _attrs(x.shape, w.shape, stride, padding, dilation, output_padding)
        pa = np.ascontiguousarray(np.asarray(pts, dtype=np.int64).reshape(-1, 2 + nd))
        xa, xp = _f64(x)
        wa, wp = _f64(w)
        ba, bp = _f64(bias)
        n = pa.shape[0]
        yv = np.empty(n, dtype=np.float64)
        sv = np.empty(n, dtype=np.float64)
        keep = [_i64(x.shape), _i64(w.shape), _i64(s), _i64(p), _i64(ph), _i64(d), _i64(op)]
        rc = self.lib.convt_oracle_points(
            nd, *[k[1] for k in keep], int(groups), xp, wp, bp, n,
            pa.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            yv.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            sv.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(nthreads))
        if rc != 0:
            raise ValueError("ill-formed problem or point out of range")
        if activation:
            yv = self.activation(activation, yv)
        return yv, sv

    def backward_data(self, dy: np.ndarray, w: np.ndarray, x_shape, stride=None, padding=None,
                      dilation=None, output_padding=None, groups: int = 1,
                      with_scale: bool = True, nthreads: int = 0):
        """Input gradient dx (shape x_shape) for the upstream gradient dy (the
        forward output's shape), in float64. Returns (dx, scale)."""
        x_shape = tuple(int(v) for v in x_shape)
        nd, s, p, ph, d, op = _attrs(x_shape, w.shape, stride, padding, dilation, output_padding)
        oshape = self.out_shape(x_shape, w.shape, s, list(zip(p, ph)), d, op, groups)
        if tuple(dy.shape) != oshape:
            raise ValueError(f"dy must have the output shape {oshape}")
        ya, yp = _f64(dy)
        wa, wp = _f64(w)
        dx = np.empty(x_shape, dtype=np.float64)
        sc = np.empty(x_shape, dtype=np.float64) if with_scale else None
        keep = [_i64(x_shape), _i64(w.shape), _i64(s), _i64(p), _i64(ph), _i64(d), _i64(op)]
        rc = self.lib.convt_oracle_backward_data(
            nd, *[k[1] for k in keep], int(groups), yp, wp,
            dx.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            sc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if sc is not None else None,
            int(nthreads))
        if rc != 0:
            raise ValueError("ill-formed transposed convolution")
        return dx, sc

    def backward_data_points(self, dy: np.ndarray, w: np.ndarray, x_shape, pts: np.ndarray,
                             stride=None, padding=None, dilation=None, output_padding=None,
                             groups: int = 1, nthreads: int = 0):
        """dx at the given points (rows of (b, ci, i...)), each on its own.
        Returns (dx, scale) as float64 arrays of length n."""
        x_shape = tuple(int(v) for v in x_shape)
        nd, s, p, ph, d, op = _attrs(x_shape, w.shape, stride, padding, dilation, output_padding)
        oshape = self.out_shape(x_shape, w.shape, s, list(zip(p, ph)), d, op, groups)
        if tuple(dy.shape) != oshape:
            raise ValueError(f"dy must have the output shape {oshape}")
        pa = np.ascontiguousarray(np.asarray(pts, dtype=np.int64).reshape(-1, 2 + nd))
        ya, yp = _f64(dy)
        wa, wp = _f64(w)
        n = pa.shape[0]
        xv = np.empty(n, dtype=np.float64)
        sv = np.empty(n, dtype=np.float64)
        keep = [_i64(x_shape), _i64(w.shape), _i64(s), _i64(p), _i64(ph), _i64(d), _i64(op)]
        rc = self.lib.convt_oracle_backward_data_points(
            nd, *[k[1] for k in keep], int(groups), yp, wp, n,
            pa.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            xv.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            sv.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(nthreads))
        if rc != 0:
            raise ValueError("ill-formed problem or point out of range")
        return xv, sv


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from this directory's source (compiled if not yet built)."""
    global _default
    if _default is None:
        # CONVT_ORACLE_LIB names another build of the same source (the
        # host-sanitizer build)
        path = os.environ.get("CONVT_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(path):
                build(force=True)
        _default = Oracle(path)
    return _default


def max_threads() -> int:
    return default().max_threads()


def out_shape(*args, **kwargs):
    return default().out_shape(*args, **kwargs)


def forward(*args, **kwargs):
    return default().forward(*args, **kwargs)


def points(*args, **kwargs):
    return default().points(*args, **kwargs)


def backward_data(*args, **kwargs):
    return default().backward_data(*args, **kwargs)


def backward_data_points(*args, **kwargs):
    return default().backward_data_points(*args, **kwargs)


def activation(*args, **kwargs):
    return default().activation(*args, **kwargs)
