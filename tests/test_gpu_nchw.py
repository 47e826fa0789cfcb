"""GPU parity of the two-byte phase GEMM that reads x in its NC[D]HW layout
(the PHASE_GEMM route for bfloat16 / float16 problems with an even input row
length and more than 64 output channels per group), against the oracle.

Shapes are chosen to reach each of the kernel's configurations (2-D kernel 4
stride 2 with 256- and 128-row channel tiles, 3-D kernel 4 stride 2, 2-D
kernel 3 stride 1 dilation 2) with ragged input channels (a partial chunk and
a padding chunk), ragged output channels (a partial channel tile), several q
tiles with masked tails, asymmetric padding and output padding. Error
measure and bounds as in tests/gpu_util.py; on integer data the outputs must
equal the oracle rounded once to the element type.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import workloads
from tests.gpu_util import TOL, check_full, oracle_full, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups
    ("k4s2_wide", (2, 72, 10, 14), (72, 136, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1),
    ("k4s2_two_co_tiles", (1, 40, 18, 34), (40, 300, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1),
    ("k4s2_narrow", (2, 48, 9, 20), (48, 100, 4, 4), (2, 2), (1, 1), (1, 1), (1, 1), 1),
    ("k4s2_groups", (1, 64, 6, 16), (64, 96, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 2),
    ("k4s2_3d", (1, 40, 5, 6, 8), (40, 100, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1),
    ("k3s1_dil2", (2, 40, 22, 26), (40, 130, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1),
    ("k3s1_dil2_pad1", (1, 24, 13, 36), (24, 72, 3, 3), (1, 1), (1, 1), (2, 2), (1, 0), 1),
    ("k4s2_asym", (1, 32, 12, 16), (32, 160, 4, 4), (2, 2), ((0, 2), (2, 1)), (1, 1), (1, 0), 1),
    ("k4s2_3d_asym", (1, 24, 4, 5, 10), (24, 80, 4, 4, 4), (2, 2, 2), ((1, 0), (0, 2), (2, 1)),
     (1, 1, 1), (0, 1, 1), 1),
    # width stride 1 with output rows of whole 16-byte pieces: the outputs
    # leave through LDS staging as 16-byte row pieces
    ("k3s1_dil2_rows24", (2, 40, 22, 24), (40, 130, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1),
    ("k3s1_rows16_groups", (2, 48, 13, 16), (48, 72, 3, 3), (1, 1), (1, 1), (1, 1), (0, 0), 2),
    ("k3s1_rows40_op", (1, 32, 9, 40), (32, 200, 3, 3), (1, 1), (1, 1), (1, 1), (0, 0), 1),
]


def tensors(case, dtype, dist, seed, bias=True):
    name, xs, ws, s, p, d, op, g = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, bias, dtype, dist, dist, dist, seed)
    return tens, dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g)


def plan_of(tens, prm, route="phase_gemm", activation="none"):
    return C.get_plan(tens.x.shape, tens.w.shape, prm["stride"], prm["padding"], prm["dilation"],
                      prm["output_padding"], prm["groups"], tens.bias is not None, tens.dtype, route,
                      activation=activation)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cases_take_the_nchw_kernel(case):
    # the planner must serve every case here with the in-place kernel (the
    # PHASE_GEMM route; PHASE_GEMM_PACKED would mean the channel-chunked copy)
    tens, prm = tensors(case, "bf16", "uniform", 1)
    assert plan_of(tens, prm, "phase_gemm").route == "phase_gemm"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_uniform(case, dtype):
    tens, prm = tensors(case, dtype, "uniform", 11)
    check_full(tens, prm, route="phase_gemm", tag=f"nchw {case[0]} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_integer_exact(case, dtype):
    tens, prm = tensors(case, dtype, "int(4)", 12)
    say(f"[gpu] nchw integer {case[0]} {dtype}")
    y, pl = run_gpu(tens, prm, "phase_gemm")
    assert pl.route == "phase_gemm"
    ref, _ = oracle_full(tens, prm)
    assert np.all(ref == np.round(ref))
    if dtype == "bf16":
        expect = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(ref.astype(np.float32)))
    else:
        expect = ref.astype(np.float16).astype(np.float32)
    bad = np.argwhere(y != expect.astype(np.float64))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("case", CASES[:3] + CASES[4:6], ids=[c[0] for c in CASES[:3] + CASES[4:6]])
def test_no_bias_and_packed_route_agree_with_oracle(case):
    # the same problems without a bias, on the in-place kernel and on the
    # channel-chunked-copy kernel
    tens, prm = tensors(case, "bf16", "normal(1)", 13, bias=False)
    check_full(tens, prm, route="phase_gemm", tag=f"nchw nobias {case[0]}")
    check_full(tens, prm, route="phase_gemm_packed", tag=f"packed nobias {case[0]}")


@pytest.mark.parametrize("act", ["relu", "sigmoid", "tanh", "silu", "gelu"])
@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[5], CASES[9], CASES[10]],
                         ids=["k4s2", "k4s2_3d", "k3s1", "k3s1_rows24", "k3s1_rows16_groups"])
def test_activations(case, act):
    # the last two store 16-byte row pieces through LDS staging: an instance
    # per activation kind on each store path
    tens, prm = tensors(case, "bf16", "uniform", 14)
    prm = dict(prm, activation=act)
    check_full(tens, prm, route="phase_gemm", tag=f"nchw {case[0]} {act}")


def test_misaligned_input_refused():
    import torch
    tens, prm = tensors(CASES[0], "bf16", "uniform", 15)
    pl = plan_of(tens, prm)
    x = to_device(tens.x_dev, "bf16")
    buf = torch.empty(x.numel() + 1, dtype=torch.bfloat16, device="cuda")
    xm = buf[1:].view(x.shape)  # 2 bytes past a 4-byte boundary
    assert xm.data_ptr() % 4 == 2
    xm.copy_(x)
    w = to_device(tens.w_dev, "bf16")
    b = to_device(tens.bias_dev, "bf16")
    say("[gpu] nchw misaligned x refused")
    with pytest.raises(C.ConvtError) as ei:
        pl.forward(xm, w, b)
    assert ei.value.status == 1
    # the packed route takes it
    pk = plan_of(tens, prm, "phase_gemm_packed")
    y = pk.forward(xm, w, b)
    torch.cuda.synchronize()
    ref, sc = oracle_full(tens, prm)
    yh = y.float().cpu().numpy().astype(np.float64)
    den = sc + np.abs(tens.bias.astype(np.float64)).reshape(1, -1, 1, 1)
    assert np.max(np.abs(yh - ref) / den) <= TOL["bf16"]
