"""GPU test of convt_forward_scratch, the forward entry point that takes no
workspace (its scratch is a fixed device array of the library): through the
C ABI it must give, byte for byte, what convt_forward gives with a caller's
workspace, on two calls in a row whose second problem is smaller, on the
routes that use a workspace (the in-place phase GEMM, its packed variant)
and on the grouped kernel, which needs none."""
import numpy as np
import pytest

import convt_forward_amd as C
import workloads
from tests.gpu_util import say, to_device, to_host64

pytestmark = pytest.mark.gpu

CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups, route
    ("gemm_2d_big", (4, 128, 16, 16), (128, 256, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, "phase_gemm"),
    ("gemm_2d_small", (1, 40, 6, 10), (40, 96, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, "phase_gemm"),
    ("packed_big", (2, 64, 12, 13), (64, 80, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, "phase_gemm_packed"),
    ("packed_small", (1, 24, 5, 7), (24, 40, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1, "phase_gemm_packed"),
    ("grouped_big", (2, 64, 16, 16), (64, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 8, "grouped"),
    ("grouped_small", (1, 32, 7, 9), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4, "grouped"),
]


def setup(case, seed):
    name, xs, ws, s, p, d, op, g, route = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, True, "bf16", "uniform", "uniform", "uniform",
                                  seed)
    pl = C.get_plan(xs, ws, s, p, d, op, g, True, "bf16", route)
    assert pl.route == route, (name, pl.route)
    # (the grouped route reads W as stored: no workspace, the scratch entry
    # point then passes none)
    assert 0 <= pl.workspace_bytes <= C.lib().convt_scratch_max_bytes()
    assert (pl.workspace_bytes == 0) == (route == "grouped")
    x, w, b = (to_device(a, "bf16") for a in (tens.x_dev, tens.w_dev, tens.bias_dev))
    return pl, x, w, b


@pytest.mark.parametrize("pair", [(0, 1), (2, 3), (4, 5), (0, 3)],
                         ids=["gemm", "packed", "grouped", "gemm_then_packed"])
def test_scratch_forward_matches_forward_two_calls(pair):
    import torch
    big, small = CASES[pair[0]], CASES[pair[1]]
    say(f"[gpu] scratch forward {big[0]} then {small[0]}")
    p1, x1, w1, b1 = setup(big, 70)
    p2, x2, w2, b2 = setup(small, 71)
    ref1 = to_host64(p1.forward(x1, w1, b1))
    ref2 = to_host64(p2.forward(x2, w2, b2))
    torch.cuda.synchronize()
    y1 = p1.new_output(x1.device).fill_(float("nan"))
    y2 = p2.new_output(x2.device).fill_(float("nan"))
    st = torch.cuda.current_stream().cuda_stream
    # two calls in a row on one stream, the second smaller
    p1.forward_scratch_ptr(x1.data_ptr(), w1.data_ptr(), b1.data_ptr(), y1.data_ptr(), st)
    p2.forward_scratch_ptr(x2.data_ptr(), w2.data_ptr(), b2.data_ptr(), y2.data_ptr(), st)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y1), ref1)
    assert np.array_equal(to_host64(y2), ref2)
    # and again, the array now holding the second call's contents
    y1.fill_(float("nan"))
    p1.forward_scratch_ptr(x1.data_ptr(), w1.data_ptr(), b1.data_ptr(), y1.data_ptr(), st)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y1), ref1)


def test_scratch_forward_full_size_generator_workload():
    import torch
    wl = workloads.get("c3")
    tens = workloads.workload_tensors(wl)
    pl = C.get_plan(wl.x_shape, wl.w_shape, wl.stride, wl.padding, wl.dilation,
                    wl.output_padding, wl.groups, True, "bf16")
    say(f"[gpu] scratch forward {wl.name}, workspace {pl.workspace_bytes} bytes")
    x, w, b = (to_device(a, "bf16") for a in (tens.x_dev, tens.w_dev, tens.bias_dev))
    ref = to_host64(pl.forward(x, w, b))
    y = pl.new_output(x.device).fill_(float("nan"))
    pl.forward_scratch_ptr(x.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y), ref)
