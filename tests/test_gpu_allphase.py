"""GPU parity of the all-phase GEMM (the PHASE_GEMM_ALLPHASE route: two-byte
types, stride 2 and dilation 1 on the height and width axes; one block
computes every (height, width) residue of an output tile, reading x and W as
stored), against the oracle.

Shapes reach both configurations (4 and 8 taps per phase: 4x4, 2x8, 4x8 and
8x4 kernels in 2-D; 4x4x4, depth stride 1, depth stride 3 and dilated depth
in 3-D) with ragged input channels (chunks of 8 past C_in/groups), ragged
output channels (a partial 128-channel tile, two tiles), groups, several q
tiles with masked tails, zero and asymmetric padding, output padding and
caller-flipped taps. Error measure and bounds as in tests/gpu_util.py; on
integer data the outputs must equal the oracle rounded once to the element
type.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import workloads
from tests.gpu_util import TOL, check_full, oracle_full, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

ROUTE = "phase_gemm_allphase"

CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups
    ("k4s2_two_co_tiles", (2, 40, 10, 16), (40, 200, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1),
    ("k4s2_ragged_ci", (1, 20, 7, 24), (20, 72, 4, 4), (2, 2), (1, 1), (1, 1), (1, 0), 1),
    ("k4s2_groups", (1, 64, 6, 16), (64, 96, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 2),
    ("k4s2_pad_h0", (2, 24, 5, 12), (24, 130, 4, 4), (2, 2), (0, 1), (1, 1), (0, 0), 1),
    ("k4s2_asym", (1, 32, 9, 16), (32, 144, 4, 4), (2, 2), ((1, 3), (0, 2)), (1, 1), (0, 0), 1),
    ("k2x8", (1, 32, 6, 10), (32, 100, 2, 8), (2, 2), (0, 1), (1, 1), (0, 0), 1),
    ("k4x8", (1, 24, 6, 8), (24, 80, 4, 8), (2, 2), (1, 3), (1, 1), (0, 0), 1),
    ("k8x4", (1, 24, 5, 12), (24, 70, 8, 4), (2, 2), (3, 1), (1, 1), (0, 0), 1),
    ("k4s2_3d", (1, 24, 4, 6, 8), (24, 72, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1),
    ("3d_depth_s1", (1, 16, 3, 6, 16), (16, 90, 2, 4, 4), (1, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1),
    ("3d_depth_s3", (1, 16, 3, 4, 8), (16, 66, 3, 4, 4), (3, 2, 2), (0, 1, 1), (1, 1, 1), (2, 0, 0), 1),
    ("3d_dil_depth", (2, 16, 3, 4, 8), (16, 66, 2, 4, 4), (1, 2, 2), (1, 1, 1), (2, 1, 1), (1, 0, 0), 1),
]


def tensors(case, dtype, dist, seed, bias=True):
    name, xs, ws, s, p, d, op, g = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, bias, dtype, dist, dist, dist, seed)
    return tens, dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g)


def plan_of(tens, prm, route=ROUTE, activation="none", flipped=False):
    return C.get_plan(tens.x.shape, tens.w.shape, prm["stride"], prm["padding"], prm["dilation"],
                      prm["output_padding"], prm["groups"], tens.bias is not None, tens.dtype, route,
                      activation=activation, taps_flipped=flipped)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cases_plan_the_allphase_kernel(case):
    tens, prm = tensors(case, "bf16", "uniform", 1)
    assert plan_of(tens, prm).route == ROUTE
    assert plan_of(tens, prm).workspace_bytes == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_uniform(case, dtype):
    tens, prm = tensors(case, dtype, "uniform", 21)
    check_full(tens, prm, route=ROUTE, tag=f"allphase {case[0]} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_integer_exact(case, dtype):
    tens, prm = tensors(case, dtype, "int(4)", 22)
    say(f"[gpu] allphase integer {case[0]} {dtype}")
    y, pl = run_gpu(tens, prm, ROUTE)
    assert pl.route == ROUTE
    ref, _ = oracle_full(tens, prm)
    assert np.all(ref == np.round(ref))
    if dtype == "bf16":
        expect = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(ref.astype(np.float32)))
    else:
        expect = ref.astype(np.float16).astype(np.float32)
    bad = np.argwhere(y != expect.astype(np.float64))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("case", CASES[:2] + CASES[5:9], ids=[c[0] for c in CASES[:2] + CASES[5:9]])
def test_no_bias_matches_the_other_gemm_routes(case):
    # the same problems without a bias, on this kernel and on the phase GEMMs
    # that run on reordered weights
    tens, prm = tensors(case, "bf16", "normal(1)", 23, bias=False)
    check_full(tens, prm, route=ROUTE, tag=f"allphase nobias {case[0]}")
    check_full(tens, prm, route="phase_gemm_packed", tag=f"packed nobias {case[0]}")


@pytest.mark.parametrize("act", ["relu", "sigmoid", "tanh", "silu", "gelu"])
@pytest.mark.parametrize("case", [CASES[0], CASES[6], CASES[8]], ids=["k4s2", "k4x8", "k4s2_3d"])
def test_activations(case, act):
    tens, prm = tensors(case, "bf16", "uniform", 24)
    prm = dict(prm, activation=act)
    check_full(tens, prm, route=ROUTE, tag=f"allphase {case[0]} {act}")


@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[6], CASES[9]],
                         ids=["k4s2", "k4s2_asym", "k4x8", "3d_depth_s1"])
def test_flipped_taps_integer_exact(case):
    # W stored spatially reversed (taps_flipped): the same outputs as the
    # forward-orientation weights
    tens, prm = tensors(case, "bf16", "int(4)", 25)
    nd = len(case[1]) - 2
    wflip = np.ascontiguousarray(np.flip(tens.w_dev, axis=tuple(range(2, 2 + nd))))
    say(f"[gpu] allphase flipped {case[0]}")
    pl = plan_of(tens, prm, flipped=True)
    assert pl.route == ROUTE
    x = to_device(tens.x_dev, "bf16")
    w = to_device(wflip, "bf16")
    b = to_device(tens.bias_dev, "bf16")
    y = pl.forward(x, w, b).float().cpu().numpy().astype(np.float64)
    ref, _ = oracle_full(tens, prm)
    expect = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(ref.astype(np.float32)))
    bad = np.argwhere(y != expect.astype(np.float64))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


def test_misaligned_weights_refused():
    import torch
    tens, prm = tensors(CASES[0], "bf16", "uniform", 26)
    pl = plan_of(tens, prm)
    x = to_device(tens.x_dev, "bf16")
    w = to_device(tens.w_dev, "bf16")
    buf = torch.empty(w.numel() + 8, dtype=torch.bfloat16, device="cuda")
    wm = buf[1:1 + w.numel()].view(w.shape)  # 2 bytes past a 16-byte boundary
    assert wm.data_ptr() % 16 == 2
    wm.copy_(w)
    b = to_device(tens.bias_dev, "bf16")
    say("[gpu] allphase misaligned W refused")
    with pytest.raises(C.ConvtError) as ei:
        pl.forward(x, wm, b)
    assert ei.value.status == 1
