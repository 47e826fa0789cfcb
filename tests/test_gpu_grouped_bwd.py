"""GPU parity of the grouped backward kernel (route_bwd GROUPED): the input
gradient of 2-D two-byte problems with few channels per group (output
channels a multiple of 8 with at most 16 (tap, 8-channel slice) slots, at
most 16 input channels per group, dy rows of whole 16-byte chunks), against
the oracle's backward data. Cases vary stride (1, 2, 3), dilation, taps
(2x2 to 4x4), channels per group (1 to 16 input, 8 and 16 output), a dx
width that is not a multiple of 4 (2-byte stores), the three filter layouts
with and without flipped taps, both two-byte types; small-integer data must
equal the oracle rounded once, uniform data meet the normalised-error bound;
a dy that is not 16-byte aligned takes the direct kernel with the same
result.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests.gpu_util import TOL, norm_error, say, to_device, to_host64
from tests.test_gpu_layouts import rearrange

pytestmark = pytest.mark.gpu

# name, x shape, W shape [C_in, C_out/groups, kh, kw], stride, padding, dilation, output_padding, groups
CASES = [
    ("cig8_cog8_k4s2", (1, 16, 32, 32), (16, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 2),
    ("cig8_g3", (2, 24, 9, 16), (24, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 3),
    ("cig16_cog16_k2", (1, 32, 6, 8), (32, 16, 2, 2), (2, 2), (0, 0), (1, 1), (0, 0), 2),
    ("s1_dil2", (1, 16, 10, 16), (16, 8, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 2),
    ("s3", (1, 8, 5, 6), (8, 8, 3, 3), (3, 3), (1, 1), (1, 1), (0, 0), 1),
    ("cig1", (1, 2, 5, 4), (2, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 2),
    ("ragged_width", (1, 16, 6, 13), (16, 8, 4, 4), (2, 2), (2, 2), (1, 1), (0, 0), 2),
]


def rne(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float64)
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v.astype(np.float32))).astype(np.float64)


def dy_tensors(case, dtype, dist, seed):
    ys = oracle.out_shape(case[1], case[2], case[3], case[4], case[5], case[6], case[7])
    return workloads.make_tensors(ys, case[2], 0, False, dtype, dist, dist, dist, seed)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_backward_integer_exact(case, dtype):
    import torch
    name, xs, ws, s, p, d, op, g = case
    pl = C.get_plan(xs, ws, s, p, d, op, g, False, dtype)
    assert pl.route_bwd == "grouped"
    t = dy_tensors(case, dtype, "int(4)", 91)
    say(f"[gpu] grouped backward {name} {dtype} integer")
    dx = pl.backward_data(to_device(t.x_dev, dtype), to_device(t.w_dev, dtype))
    torch.cuda.synchronize()
    ref, _ = oracle.backward_data(t.x, t.w, xs, s, p, d, op, g, with_scale=False)
    bad = np.argwhere(to_host64(dx) != rne(ref, dtype))
    assert bad.size == 0, f"{name} {dtype}: {len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_backward_uniform(case, dtype):
    import torch
    name, xs, ws, s, p, d, op, g = case
    pl = C.get_plan(xs, ws, s, p, d, op, g, False, dtype, "auto", "grouped")
    t = dy_tensors(case, dtype, "uniform", 92)
    say(f"[gpu] grouped backward {name} {dtype} uniform")
    dx = pl.backward_data(to_device(t.x_dev, dtype), to_device(t.w_dev, dtype))
    torch.cuda.synchronize()
    ref, sc = oracle.backward_data(t.x, t.w, xs, s, p, d, op, g)
    e = norm_error(to_host64(dx), ref, sc, np.zeros(ref.shape), dtype=dtype)
    assert e <= TOL[dtype], f"{name} {dtype}: error {e}"


@pytest.mark.parametrize("flipped", [False, True])
@pytest.mark.parametrize("layout", ["ci_co_k", "k_ci_co", "k_co_ci"])
@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4]], ids=[CASES[0][0], CASES[2][0], CASES[4][0]])
def test_grouped_backward_filter_layouts(case, layout, flipped):
    import torch
    name, xs, ws, s, p, d, op, g = case
    pl = C.get_plan(xs, ws, s, p, d, op, g, False, "bf16", "auto", "grouped", layout, flipped)
    assert pl.route_bwd == "grouped"
    t = dy_tensors(case, "bf16", "int(4)", 93)
    say(f"[gpu] grouped backward {name} layout {layout} flipped={flipped}")
    w = to_device(rearrange(t.w_dev, g, layout, flipped), "bf16")
    dx = pl.backward_data(to_device(t.x_dev, "bf16"), w)
    torch.cuda.synchronize()
    ref, _ = oracle.backward_data(t.x, t.w, xs, s, p, d, op, g, with_scale=False)
    bad = np.argwhere(to_host64(dx) != rne(ref, "bf16"))
    assert bad.size == 0, f"{name} {layout} flipped={flipped}: {len(bad)} mismatches, first at {bad[0]}"


def test_grouped_backward_unaligned_dy_takes_direct_kernel():
    import torch
    case = CASES[1]
    name, xs, ws, s, p, d, op, g = case
    pl = C.get_plan(xs, ws, s, p, d, op, g, False, "bf16")
    assert pl.route_bwd == "grouped"
    t = dy_tensors(case, "bf16", "int(4)", 94)
    dy_al = to_device(t.x_dev, "bf16")
    # the same values 2 bytes into a larger buffer: not 16-byte aligned
    big = torch.zeros(dy_al.numel() + 8, dtype=torch.bfloat16, device="cuda")
    dy = big[1:1 + dy_al.numel()].view(dy_al.shape)
    dy.copy_(dy_al)
    assert dy.data_ptr() % 16 != 0
    say(f"[gpu] grouped backward {name} with dy at {dy.data_ptr():#x}")
    dx = pl.backward_data(dy, to_device(t.w_dev, "bf16"))
    torch.cuda.synchronize()
    ref, _ = oracle.backward_data(t.x, t.w, xs, s, p, d, op, g, with_scale=False)
    bad = np.argwhere(to_host64(dx) != rne(ref, "bf16"))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"
