"""GPU parity of the filter layouts and caller-flipped taps (the AWS Neuron
conv3d_transpose page's filter_shape and flip_filter_taps_in_kernel; element
(ci, ocl, kk) per include/convt.h): W is rearranged on the host from the
[C_in, C_out/groups, k...] forward-orientation array the oracle takes, and
every route, forward and backward data, must give the oracle's result. The
data are small integers, so float32 results are exact and bfloat16 results
equal the oracle rounded once to bfloat16.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests.gpu_util import say, to_device, to_host64

pytestmark = pytest.mark.gpu


def rearrange(w: np.ndarray, groups: int, layout: str, flipped: bool) -> np.ndarray:
    """W [C_in, Cog, k...] in `layout`, spatially reversed when `flipped`."""
    nd = w.ndim - 2
    if flipped:
        w = w[(slice(None), slice(None)) + (slice(None, None, -1),) * nd]
    if layout == "ci_co_k":
        out = w
    elif layout == "k_ci_co":
        out = np.moveaxis(w, (0, 1), (nd, nd + 1))
    else:  # k_co_ci: element (kk, g*Cog + ocl, cil) = W[g*Cig + cil, ocl, kk]
        ci, cog = w.shape[:2]
        wg = w.reshape((groups, ci // groups, cog) + w.shape[2:])
        out = np.moveaxis(wg, (0, 1, 2), (nd, nd + 2, nd + 1)).reshape(
            w.shape[2:] + (groups * cog, ci // groups))
    # a copy: a flipped size-1 axis keeps a negative stride that numpy still
    # calls contiguous (and torch.from_numpy refuses)
    return np.array(out, order="C", copy=True)


def rne_bf16(v):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v.astype(np.float32))).astype(
        np.float64)


CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups, dtype
    ("c1_like_f32", (2, 4, 8, 8), (4, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1, "f32"),
    ("c3_like_bf16", (2, 72, 9, 13), (72, 136, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, "bf16"),
    ("c4a_like_bf16", (2, 32, 7, 9), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4, "bf16"),
    ("grouped_3d_f32", (1, 12, 3, 4, 5), (12, 4, 3, 2, 2), (2, 1, 2), (1, 0, 1), (1, 1, 1),
     (1, 0, 0), 3, "f32"),
    ("dilated_1d_bf16", (2, 40, 37), (40, 24, 5), (3,), (2,), (2,), (1,), 2, "bf16"),
]
COMBOS = [(lay, fl) for lay in ("ci_co_k", "k_ci_co", "k_co_ci") for fl in (False, True)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("layout,flipped", COMBOS, ids=[f"{l}{'-flip' if f else ''}" for l, f in COMBOS])
def test_filter_layouts_forward_and_backward(case, layout, flipped):
    import torch
    name, xs, ws, s, p, d, op, g, dt = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, True, dt, "int(4)", "int(4)", "int(4)", 90)
    ref, _ = oracle.forward(tens.x, tens.w, tens.bias, s, p, d, op, g, with_scale=False)
    expect = ref if dt == "f32" else rne_bf16(ref)
    x = to_device(tens.x_dev, dt)
    b = to_device(tens.bias_dev, dt)
    w = to_device(rearrange(tens.w_dev, g, layout, flipped), dt)
    for route in ["auto", "naive", "direct", "phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "grouped"]:
        try:
            pl = C.get_plan(xs, ws, s, p, d, op, g, True, dt, route, "auto", layout, flipped)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        say(f"[gpu] layout {layout} flipped={flipped} {name} forward route={pl.route}")
        y = pl.forward(x, w, b)
        torch.cuda.synchronize()
        got = to_host64(y)
        bad = np.argwhere(got != expect)
        assert bad.size == 0, f"forward {route}: {len(bad)} mismatches, first at {bad[0]}"
    # backward data
    dyt = workloads.make_tensors(ref.shape, ws, 0, False, dt, "int(4)", "int(4)", "int(4)", 91)
    dref, _ = oracle.backward_data(dyt.x, tens.w, xs, s, p, d, op, g, with_scale=False)
    dexp = dref if dt == "f32" else rne_bf16(dref)
    dy = to_device(dyt.x_dev, dt)
    for route in ["auto", "naive", "phase_gemm", "direct"]:
        try:
            pl = C.get_plan(xs, ws, s, p, d, op, g, False, dt, "auto", route, layout, flipped)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        say(f"[gpu] layout {layout} flipped={flipped} {name} backward route={pl.route_bwd}")
        dx = pl.backward_data(dy, w)
        torch.cuda.synchronize()
        bad = np.argwhere(to_host64(dx) != dexp)
        assert bad.size == 0, f"backward {route}: {len(bad)} mismatches, first at {bad[0]}"
