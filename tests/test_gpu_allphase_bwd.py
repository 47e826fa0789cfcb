"""GPU parity of the backward all-phase GEMM (route_bwd phase_gemm_allphase:
two-byte types, stride 2 and dilation 1 on the height and width axes with 16
taps over the two; dy and W read as stored, four phase planes per halo)
against the oracle's input gradient.

Both of the kernel's tilings run: the first case keeps the 256-position box,
the others take the K split. Shapes reach every tap layout the kernel takes (4x4, 2x8, 8x2; 3-D with
depth stride 1, 2 and 3 and a dilated depth) with ragged dx channel tiles
(128-channel tiles past C_in/groups), ragged dy channel chunks (8 channels
past C_out/groups, an odd chunk count), groups, boxes with masked tails
(16-, 32- and 64-wide), even and odd, zero and asymmetric padding, output padding
and caller-flipped taps. Error measure and bounds as in tests/gpu_util.py; on
integer data the dx values must equal the oracle rounded once to the element
type.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests.gpu_util import TOL, norm_error, say, to_device, to_host64
from tests.test_gpu_backward import bwd_tensors, rne_bf16

pytestmark = pytest.mark.gpu

ROUTE = "phase_gemm_allphase"

CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups
    # 160 blocks of 256-position boxes (with the K split 320, two rounds of
    # the GPU): the planner keeps the full box; every case below is small
    # enough for the K split (128-position boxes, two wave pairs per stage)
    ("k4s2_full_box", (40, 512, 16, 16), (512, 16, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1),
    ("k4s2_two_ci_tiles", (2, 200, 10, 16), (200, 40, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1),
    ("k4s2_ragged_cog", (1, 72, 7, 24), (72, 20, 4, 4), (2, 2), (1, 1), (1, 1), (1, 0), 1),
    ("k4s2_groups", (1, 192, 6, 16), (192, 24, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 2),
    ("k4s2_pad_0_2", (2, 130, 5, 8), (130, 24, 4, 4), (2, 2), (0, 2), (1, 1), (0, 0), 1),
    ("k4s2_asym", (1, 144, 9, 16), (144, 32, 4, 4), (2, 2), ((1, 3), (0, 2)), (1, 1), (0, 0), 1),
    ("k2x8", (1, 100, 6, 16), (100, 32, 2, 8), (2, 2), (0, 3), (1, 1), (0, 0), 1),
    ("k8x2", (1, 70, 5, 24), (70, 24, 8, 2), (2, 2), (3, 1), (1, 1), (0, 0), 1),
    ("k4s2_wide_rows", (1, 80, 12, 40), (80, 24, 4, 4), (2, 2), (1, 1), (1, 1), (1, 0), 1),
    ("k4s2_rows64_pad2", (1, 80, 4, 64), (80, 16, 4, 4), (2, 2), (2, 2), (1, 1), (0, 0), 1),
    ("k4s2_3d", (1, 72, 4, 6, 8), (72, 24, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1),
    ("3d_depth_s1", (1, 90, 3, 6, 16), (90, 16, 2, 4, 4), (1, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1),
    ("3d_depth_s3", (1, 66, 3, 4, 8), (66, 16, 3, 4, 4), (3, 2, 2), (0, 1, 1), (1, 1, 1), (2, 0, 0), 1),
    ("3d_dil_depth", (2, 66, 3, 4, 8), (66, 16, 2, 4, 4), (1, 2, 2), (1, 1, 1), (2, 1, 1), (1, 0, 0), 1),
]


def prm_of(case):
    return dict(stride=case[3], padding=case[4], dilation=case[5], output_padding=case[6],
                groups=case[7])


def plan_of(case, dtype="bf16", route_bwd=ROUTE, flipped=False):
    prm = prm_of(case)
    return C.get_plan(case[1], case[2], prm["stride"], prm["padding"], prm["dilation"],
                      prm["output_padding"], prm["groups"], False, dtype, "auto", route_bwd,
                      taps_flipped=flipped)


def run(case, dtype, dist, seed, flipped=False):
    import torch
    prm = prm_of(case)
    tens = bwd_tensors(case[1], case[2], prm, dtype, dist, seed)
    pl = plan_of(case, dtype, flipped=flipped)
    assert pl.route_bwd == ROUTE
    wd = tens.w_dev
    if flipped:
        nd = len(case[1]) - 2
        wd = np.ascontiguousarray(np.flip(wd, axis=tuple(range(2, 2 + nd))))
    dy = to_device(tens.x_dev, dtype)
    w = to_device(wd, dtype)
    dx = pl.backward_data(dy, w)
    torch.cuda.synchronize()
    ref, sc = oracle.backward_data(tens.x, tens.w, case[1], prm["stride"], prm["padding"],
                                   prm["dilation"], prm["output_padding"], prm["groups"])
    return to_host64(dx), ref, sc


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_uniform(case, dtype):
    say(f"[gpu] bwd allphase {case[0]} {dtype}")
    dx, ref, sc = run(case, dtype, "uniform", 81)
    assert dx.shape == ref.shape
    e = norm_error(dx, ref, sc, np.zeros_like(sc), dtype=dtype)
    say(f"[gpu]   -> max normalised error {e:.3e}")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_integer_exact(case, dtype):
    say(f"[gpu] bwd allphase integer {case[0]} {dtype}")
    dx, ref, _ = run(case, dtype, "int(4)", 82)
    assert np.all(ref == np.round(ref))
    expect = rne_bf16(ref) if dtype == "bf16" else ref.astype(np.float16).astype(np.float64)
    bad = np.argwhere(dx != expect)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("case", [CASES[1], CASES[5], CASES[6], CASES[10]],
                         ids=["k4s2", "k4s2_asym", "k2x8", "3d_depth_s1"])
def test_flipped_taps_integer_exact(case):
    # W stored spatially reversed (taps_flipped): the same dx
    say(f"[gpu] bwd allphase flipped {case[0]}")
    dx, ref, _ = run(case, "bf16", "int(4)", 83, flipped=True)
    bad = np.argwhere(dx != rne_bf16(ref))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


def test_matches_the_phase_gemm_route():
    # the same problem on the backward phase GEMM (reordered weights,
    # channel-chunked dy copy): both within the bound of the oracle
    import torch
    case = CASES[1]
    prm = prm_of(case)
    tens = bwd_tensors(case[1], case[2], prm, "bf16", "normal(1)", 84)
    ref, sc = oracle.backward_data(tens.x, tens.w, case[1], prm["stride"], prm["padding"],
                                   prm["dilation"], prm["output_padding"], prm["groups"])
    dy = to_device(tens.x_dev, "bf16")
    w = to_device(tens.w_dev, "bf16")
    for route in [ROUTE, "phase_gemm"]:
        pl = plan_of(case, route_bwd=route)
        say(f"[gpu] bwd {route} {case[0]} normal(1)")
        dx = pl.backward_data(dy, w)
        torch.cuda.synchronize()
        e = norm_error(to_host64(dx), ref, sc, np.zeros_like(sc), dtype="bf16")
        assert e <= TOL["bf16"], f"{route}: {e}"


def test_misaligned_pointers_refused():
    import torch
    case = CASES[1]
    prm = prm_of(case)
    tens = bwd_tensors(case[1], case[2], prm, "bf16", "uniform", 85)
    pl = plan_of(case)
    dy = to_device(tens.x_dev, "bf16")
    w = to_device(tens.w_dev, "bf16")
    buf = torch.empty(w.numel() + 8, dtype=torch.bfloat16, device="cuda")
    wm = buf[1:1 + w.numel()].view(w.shape)  # 2 bytes past a 16-byte boundary
    wm.copy_(w)
    say("[gpu] bwd allphase misaligned W refused")
    with pytest.raises(C.ConvtError) as ei:
        pl.backward_data(dy, wm)
    assert ei.value.status == 1
    dxb = torch.empty(int(np.prod(case[1])) + 8, dtype=torch.bfloat16, device="cuda")
    dxm = dxb[4:4 + int(np.prod(case[1]))].view(case[1])  # 8 bytes past a 16-byte boundary
    with pytest.raises(C.ConvtError) as ei:
        pl.backward_data(dy, w, dx=dxm)
    assert ei.value.status == 1
