"""Helpers of the GPU parity tests: run the HIP path through the C ABI on seeded
host buffers and measure its error against the oracle.

Parity criterion (per output element, over the compared outputs):
    e = |y_gpu - y_ref| / (scale + |bias[oc]|)
where scale is the oracle's sum of |x * W| over the output's terms. The bias
is one more term of the sum, so it joins the denominator; outputs whose
denominator is 0 (no terms, no bias) must be exactly 0. Bounds: 1e-5 for
float32, 1e-2 for bfloat16 inputs (float32 accumulation, one rounding of the
output to bfloat16 contributes up to 2^-9).
"""
from __future__ import annotations

import sys

import numpy as np

import convt_forward_amd as C
import oracle
import workloads

# float16: one rounding of the output (2^-11 of its magnitude, which the
# denominator bounds) plus float32 accumulation: 1e-3
TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 1e-3}
# A rounding into the subnormal range errs by up to half the subnormal
# spacing, an absolute amount that the relative bounds above do not cover
# (a float16 output of 2.1e-5 = one product x*w, rounded once, is off by
# 1.06e-3 of itself): the error measure subtracts this floor first. float16
# 2^-25, bfloat16 2^-134, float32 2^-150.
SUBNORMAL_FLOOR = {"f32": 2.0 ** -150, "bf16": 2.0 ** -134, "f16": 2.0 ** -25}
# Lipschitz constant of each activation (convt_activation code): with an
# activation f the denominator becomes L_f * (scale + |bias|) + |f(y_ref)|,
# the bound on the pre-activation error carried through f plus the rounding
# of f's value
ACT_LIPSCHITZ = {0: 1.0, 1: 1.0, 2: 0.25, 3: 1.0, 4: 1.1, 5: 1.13}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    a = np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.float16 if dtype == "f16" else torch.bfloat16)


def to_host64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(tens: workloads.Tensors, params: dict, route: str = "auto", stream=None):
    """y on the GPU (as float64 numpy) and the plan that produced it."""
    import torch
    x = to_device(tens.x_dev, tens.dtype)
    w = to_device(tens.w_dev, tens.dtype)
    b = to_device(tens.bias_dev, tens.dtype) if tens.bias is not None else None
    pl = C.get_plan(tuple(x.shape), tuple(w.shape), params["stride"], params["padding"],
                    params["dilation"], params["output_padding"], params["groups"], b is not None,
                    tens.dtype, route, activation=params.get("activation", "none"))
    y = pl.forward(x, w, b, stream=stream)
    torch.cuda.synchronize()
    return to_host64(y), pl


def params_of(wl: workloads.Workload) -> dict:
    return dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation,
                output_padding=wl.output_padding, groups=wl.groups)


def oracle_full(tens: workloads.Tensors, params: dict):
    """(y, scale): y after the activation, scale the magnitude sum of the
    terms before it."""
    return oracle.forward(tens.x, tens.w, tens.bias, params["stride"], params["padding"],
                          params["dilation"], params["output_padding"], params["groups"],
                          activation=C.ACTIVATIONS[params.get("activation", "none")])


def norm_error(y_gpu: np.ndarray, y_ref: np.ndarray, scale: np.ndarray, bias_abs: np.ndarray,
               act: int = 0, dtype: str | None = None):
    """max normalised error; outputs with zero denominator must match exactly.
    With an activation, the denominator is L_f * (scale + |bias|) + |y_ref|.
    With the element type given, the error first loses the type's subnormal
    rounding floor (SUBNORMAL_FLOOR)."""
    den = scale + bias_abs
    if act:
        den = ACT_LIPSCHITZ[act] * den + np.abs(y_ref)
    diff = np.abs(y_gpu - y_ref)
    zero = den == 0
    if np.any(zero) and np.any(diff[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    if dtype is not None:
        diff = np.maximum(diff - SUBNORMAL_FLOOR[dtype], 0.0)
    return float(np.max(diff[~zero] / den[~zero]))


def bias_abs_full(tens: workloads.Tensors, shape) -> np.ndarray:
    nd = len(shape) - 2
    if tens.bias is None:
        return np.zeros(shape)
    return np.broadcast_to(np.abs(tens.bias.astype(np.float64)).reshape((1, -1) + (1,) * nd), shape)


def check_full(tens, params, route="auto", tag=""):
    say(f"[gpu] {tag} route={route} x={tens.x.shape} w={tens.w.shape} {params} {tens.dtype}")
    y, pl = run_gpu(tens, params, route)
    ref, sc = oracle_full(tens, params)
    assert y.shape == ref.shape
    e = norm_error(y, ref, sc, bias_abs_full(tens, ref.shape),
                   C.ACTIVATIONS[params.get("activation", "none")], tens.dtype)
    say(f"[gpu]   -> plan route {pl.route}, max normalised error {e:.3e}")
    assert e <= TOL[tens.dtype], f"{tag}: error {e} above {TOL[tens.dtype]}"
    return y, ref, pl


def sample_points(shape, rng, n_random=20000):
    """Random outputs plus whole rows at the edges of a few planes."""
    nd = len(shape) - 2
    pts = [np.stack([rng.integers(0, s, n_random) for s in shape], axis=1)]
    sp = shape[2:]
    for b, oc in [(0, 0), (shape[0] - 1, shape[1] - 1), (shape[0] // 2, shape[1] // 2)]:
        # first and last row of the plane (along the last axis), all positions
        for lead in [(0,) * (nd - 1), tuple(s - 1 for s in sp[:-1])]:
            row = np.array([(b, oc) + lead + (w,) for w in range(sp[-1])], dtype=np.int64)
            pts.append(row)
        # first and last column
        if nd >= 2:
            for wv in (0, sp[-1] - 1):
                col = np.array([(b, oc) + (0,) * (nd - 2) + (h, wv) for h in range(sp[-2])],
                               dtype=np.int64)
                pts.append(col)
    return np.concatenate(pts, axis=0).astype(np.int64)


def check_sampled(y: np.ndarray, tens, params, pts):
    yv, sv = oracle.points(tens.x, tens.w, tens.bias, pts, params["stride"], params["padding"],
                           params["dilation"], params["output_padding"], params["groups"])
    got = y[tuple(pts.T)]
    babs = np.abs(tens.bias[pts[:, 1]].astype(np.float64)) if tens.bias is not None else 0.0 * yv
    return norm_error(got, yv, sv, babs, dtype=tens.dtype), got, yv
