"""GPU parity of the grouped kernel's segment-pair instance.

The host picks that instance when every item takes the segment-pair path:
width stride 2, at most 8 output channels per group, a q width of whole
16-position segment pairs, every phase's (tap, 8-channel slice) slots filling
its MFMA K steps, and y rows of whole 16-byte pieces. Every problem here
meets those conditions (q width 32, output rows of 64 two-byte values, 16-byte
aligned torch allocations), so the instance runs; they vary what it must get
right: fewer than 8 channels per group (padding columns), two slices per tap
(two K steps), a 3-D problem, each activation in both two-byte types, and the
three filter layouts with and without flipped taps (the kernel gathers its
MFMA weight fragments from W as stored). Small-integer data must equal the oracle
rounded once; uniform data must meet the normalised-error bound.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests.gpu_util import check_full, say, to_device, to_host64
from tests.test_gpu_layouts import rearrange

pytestmark = pytest.mark.gpu

# name, x shape, W shape [C_in, C_out/groups, k...], stride, padding, dilation, output_padding, groups
CASES = [
    ("cig8_cog8", (2, 32, 16, 32), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4),
    ("cig8_cog4", (2, 16, 8, 32), (16, 4, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 2),
    ("cig16_cog8", (2, 64, 8, 32), (64, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4),
    ("video_3d", (1, 16, 4, 6, 32), (16, 8, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 2),
]


def rne(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float64)
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v.astype(np.float32))).astype(np.float64)


def params(case, activation="none"):
    return dict(stride=case[3], padding=case[4], dilation=case[5], output_padding=case[6],
                groups=case[7], activation=activation)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_segment_pairs_integer_exact(case, dtype):
    import torch
    name, xs, ws, s, p, d, op, g = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, True, dtype, "int(4)", "int(4)", "int(4)", 81)
    pl = C.get_plan(xs, ws, s, p, d, op, g, True, dtype, "grouped")
    assert pl.route == "grouped"
    say(f"[gpu] segment pairs {name} {dtype} integer")
    y = pl.forward(to_device(tens.x_dev, dtype), to_device(tens.w_dev, dtype), to_device(tens.bias_dev, dtype))
    torch.cuda.synchronize()
    ref, _ = oracle.forward(tens.x, tens.w, tens.bias, s, p, d, op, g, with_scale=False)
    bad = np.argwhere(to_host64(y) != rne(ref, dtype))
    assert bad.size == 0, f"{name} {dtype}: {len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("act", ["relu", "sigmoid", "tanh", "silu", "gelu"])
def test_segment_pairs_activation(act, dtype):
    case = CASES[0]
    tens = workloads.make_tensors(case[1], case[2], case[2][1] * case[7], True, dtype, "uniform", "uniform",
                                  "uniform", 82)
    _, _, pl = check_full(tens, params(case, act), route="grouped", tag=f"segment pairs {act} {dtype}")
    assert pl.route == "grouped"


@pytest.mark.parametrize("flipped", [False, True])
@pytest.mark.parametrize("layout", ["ci_co_k", "k_ci_co", "k_co_ci"])
@pytest.mark.parametrize("case", [CASES[0], CASES[2]], ids=[CASES[0][0], CASES[2][0]])
def test_segment_pairs_filter_layouts(case, layout, flipped):
    import torch
    name, xs, ws, s, p, d, op, g = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, True, "bf16", "int(4)", "int(4)", "int(4)", 83)
    pl = C.get_plan(xs, ws, s, p, d, op, g, True, "bf16", "grouped", "auto", layout, flipped)
    assert pl.route == "grouped"
    say(f"[gpu] segment pairs {name} layout {layout} flipped={flipped}")
    w = to_device(rearrange(tens.w_dev, g, layout, flipped), "bf16")
    y = pl.forward(to_device(tens.x_dev, "bf16"), w, to_device(tens.bias_dev, "bf16"))
    torch.cuda.synchronize()
    ref, _ = oracle.forward(tens.x, tens.w, tens.bias, s, p, d, op, g, with_scale=False)
    bad = np.argwhere(to_host64(y) != rne(ref, "bf16"))
    assert bad.size == 0, f"{name} {layout} flipped={flipped}: {len(bad)} mismatches, first at {bad[0]}"
