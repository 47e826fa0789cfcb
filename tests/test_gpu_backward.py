"""GPU parity of the backward-data pass (dx from dy) against the oracle's
input gradient, through the C ABI.

Error measure as for the forward (tests/gpu_util.py): per dx element
|dx_gpu - dx_ref| / scale, scale the oracle's sum of |dy * W| over the
element's terms (no bias enters), bounds 1e-5 (float32) and 1e-2 (bfloat16
inputs, float32 accumulation, one rounding). On integer data every partial
sum is an integer below 2^24, so float32 results must equal the oracle and
bfloat16 results the oracle rounded once to bfloat16.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests import oracle_pins
from tests.gpu_util import TOL, norm_error, say, to_device, to_host64

pytestmark = pytest.mark.gpu

ROUTES = ["auto", "naive", "phase_gemm", "direct", "phase_gemm_allphase", "grouped"]


def bwd_tensors(xs, ws, prm, dtype, dist, seed):
    """Seeded dy (the forward output's shape) and W, as a Tensors record
    whose x field holds dy."""
    ys = oracle.out_shape(xs, ws, prm["stride"], prm["padding"], prm["dilation"],
                          prm["output_padding"], prm["groups"])
    return workloads.make_tensors(ys, ws, 0, False, dtype, dist, dist, dist, seed)


def run_bwd(tens, xs, prm, route="auto"):
    import torch
    dy = to_device(tens.x_dev, tens.dtype)
    w = to_device(tens.w_dev, tens.dtype)
    pl = C.get_plan(tuple(xs), tuple(w.shape), prm["stride"], prm["padding"], prm["dilation"],
                    prm["output_padding"], prm["groups"], False, tens.dtype, "auto", route)
    dx = pl.backward_data(dy, w)
    torch.cuda.synchronize()
    return to_host64(dx), pl


def plan_or_skip(xs, ws, prm, dtype, route):
    try:
        return C.get_plan(tuple(xs), tuple(ws), prm["stride"], prm["padding"], prm["dilation"],
                          prm["output_padding"], prm["groups"], False, dtype, "auto", route)
    except C.ConvtError as e:
        assert e.status == 2
        pytest.skip(f"route {route} does not serve this problem")


def check_bwd_full(xs, ws, prm, dtype, route, seed, tag):
    plan_or_skip(xs, ws, prm, dtype, route)
    tens = bwd_tensors(xs, ws, prm, dtype, "uniform", seed)
    say(f"[gpu] bwd {tag} route={route} x={xs} w={ws} {prm} {dtype}")
    dx, pl = run_bwd(tens, xs, prm, route)
    ref, sc = oracle.backward_data(tens.x, tens.w, xs, prm["stride"], prm["padding"],
                                   prm["dilation"], prm["output_padding"], prm["groups"])
    assert dx.shape == ref.shape
    e = norm_error(dx, ref, sc, np.zeros_like(sc), dtype=dtype)
    say(f"[gpu]   -> plan route {pl.route_bwd}, max normalised error {e:.3e}")
    assert e <= TOL[dtype], f"{tag}: error {e}"


def rne_bf16(v: np.ndarray) -> np.ndarray:
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v.astype(np.float32))).astype(
        np.float64)


def check_bwd_integer(xs, ws, prm, dtype, route, seed, tag):
    plan_or_skip(xs, ws, prm, dtype, route)
    tens = bwd_tensors(xs, ws, prm, dtype, "int(4)", seed)
    say(f"[gpu] bwd integer {tag} route={route}")
    dx, _ = run_bwd(tens, xs, prm, route)
    ref, _ = oracle.backward_data(tens.x, tens.w, xs, prm["stride"], prm["padding"],
                                  prm["dilation"], prm["output_padding"], prm["groups"])
    expect = ref if dtype == "f32" else rne_bf16(ref)
    bad = np.argwhere(dx != expect)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


# Reduced versions of the workloads (same attributes), spanning several tiles
# with ragged tails, plus asymmetric padding and grouped problems.
CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups, dtype
    ("c1_like_f32", (2, 4, 8, 8), (4, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1, "f32"),
    ("c2_like_f32", (2, 40, 300), (40, 24, 8), (4,), (2,), (1,), (0,), 1, "f32"),
    ("c3_like_bf16", (2, 72, 9, 13), (72, 136, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, "bf16"),
    ("c3_like_f32", (2, 40, 9, 13), (40, 70, 4, 4), (2, 2), (1, 1), (1, 1), (1, 0), 1, "f32"),
    ("c4a_like_bf16", (2, 32, 7, 9), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4, "bf16"),
    ("c4b_like_bf16", (2, 40, 11, 13), (40, 40, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1, "bf16"),
    ("c5_like_bf16", (1, 40, 3, 5, 7), (40, 24, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1),
     (0, 0, 0), 1, "bf16"),
    ("asym_bf16", (2, 24, 6, 7), (24, 40, 3, 3), (2, 2), ((0, 2), (2, 1)), (1, 1), (1, 0), 1,
     "bf16"),
    ("stride3_dil2_f32", (1, 12, 5, 9), (12, 20, 3, 4), (3, 2), (2, 1), (2, 1), (1, 1), 1, "f32"),
]


def case_prm(c):
    return dict(stride=c[3], padding=c[4], dilation=c[5], output_padding=c[6], groups=c[7])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("route", ROUTES)
def test_backward_data_reduced(case, route):
    check_bwd_full(case[1], case[2], case_prm(case), case[8], route, 70, f"{case[0]}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("route", ROUTES)
def test_backward_data_integer_exact(case, route):
    check_bwd_integer(case[1], case[2], case_prm(case), case[8], route, 71, f"{case[0]}")


def grid_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for prm in oracle_pins.random_grid(rng, n):
        prm = dict(prm)
        prm["Ci"] *= int(rng.choice([1, 1, 4, 12]))
        prm["Cog"] = int(prm["Cog"] * int(rng.choice([1, 3, 20])))
        prm["dtype"] = str(rng.choice(["f32", "bf16"]))
        prm["seed"] = int(rng.integers(0, 2**31))
        out.append(prm)
    return out


GRID = grid_cases(40, 4242)


@pytest.mark.parametrize("idx", range(len(GRID)))
def test_backward_data_random_grid(idx):
    prm = GRID[idx]
    xs = (prm["B"], prm["Ci"]) + tuple(prm["I"])
    ws = (prm["Ci"], prm["Cog"]) + tuple(prm["k"])
    pad = tuple(prm["p"]) if prm["p"] == prm["ph"] else tuple(zip(prm["p"], prm["ph"]))
    p = dict(stride=tuple(prm["s"]), padding=pad, dilation=tuple(prm["d"]),
             output_padding=tuple(prm["op"]), groups=prm["groups"])
    for route in ROUTES:
        try:
            C.get_plan(xs, ws, p["stride"], p["padding"], p["dilation"], p["output_padding"],
                       p["groups"], False, prm["dtype"], "auto", route)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        check_bwd_full(xs, ws, p, prm["dtype"], route, prm["seed"], f"grid[{idx}]")


# The workloads at full size (dy drawn like each workload's input), in the
# launch configuration the benchmark's backward leg times: every dx element
# against the oracle's full input gradient.
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4a", "c4b", "c5"])
def test_backward_data_workloads_all_outputs(name):
    wl = workloads.get(name)
    prm = dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation,
               output_padding=wl.output_padding, groups=wl.groups)
    tens = bwd_tensors(wl.x_shape, wl.w_shape, prm, wl.dtype, wl.x_dist, wl.seed + 1000)
    say(f"[gpu] bwd {name} full size, all outputs")
    dx, pl = run_bwd(tens, wl.x_shape, prm)
    ref, sc = oracle.backward_data(tens.x, tens.w, wl.x_shape, prm["stride"], prm["padding"],
                                   prm["dilation"], prm["output_padding"], prm["groups"])
    assert dx.shape == ref.shape
    e = norm_error(dx, ref, sc, np.zeros_like(sc), dtype=wl.dtype)
    say(f"[gpu]   -> route {pl.route_bwd}, max normalised error {e:.3e}")
    assert e <= TOL[wl.dtype]


def test_backward_data_edge_cases():
    import torch
    # no output channels: dx = 0 (fill route)
    xs, ws = (2, 3, 5), (3, 0, 3)
    prm = dict(stride=(2,), padding=(1,), dilation=(1,), output_padding=(0,), groups=1)
    say("[gpu] bwd no output channels")
    pl = C.get_plan(xs, ws, (2,), (1,), (1,), (0,), 1, False, "f32")
    assert pl.route_bwd == "fill"
    dy = torch.empty(pl.out_shape, dtype=torch.float32, device="cuda")
    w = torch.empty(ws, dtype=torch.float32, device="cuda")
    dx = torch.full(xs, 7.0, dtype=torch.float32, device="cuda")
    pl.backward_data(dy, w, dx=dx)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx).item() == 0
    # empty batch: nothing to do
    pl = C.get_plan((0, 3, 5), (3, 2, 3), (2,), (1,), (1,), (0,), 1, False, "f32")
    assert pl.route_bwd == "none"
    del prm


def test_backward_data_large_plane_sampled():
    """dy planes of 5792^2 positions (1 GiB channel-chunked copy): sampled
    dx elements on every backward route."""
    import torch
    xs, ws = (1, 8, 2896, 2896), (8, 8, 3, 3)
    prm = dict(stride=(2, 2), padding=(1, 1), dilation=(1, 1), output_padding=(1, 1), groups=1)
    t = bwd_tensors(xs, ws, prm, "bf16", "uniform", 78)
    dy = to_device(t.x_dev, "bf16")
    w = to_device(t.w_dev, "bf16")
    rng = np.random.default_rng(104)
    pts = np.stack([rng.integers(0, v, 20000) for v in xs], axis=1).astype(np.int64)
    xv, sv = oracle.backward_data_points(t.x, t.w, xs, pts, **prm)
    for route in ["auto", "phase_gemm", "naive"]:
        pl = C.get_plan(xs, ws, prm["stride"], prm["padding"], prm["dilation"],
                        prm["output_padding"], 1, False, "bf16", "auto", route)
        say(f"[gpu] bwd large plane route={pl.route_bwd}")
        dx = pl.backward_data(dy, w)
        torch.cuda.synchronize()
        got = to_host64(dx[tuple(torch.from_numpy(pts.T).to(dx.device))])
        e = norm_error(got, xv, sv, np.zeros_like(sv), dtype="bf16")
        assert e <= TOL["bf16"], f"{route}: {e}"
        del dx
        torch.cuda.empty_cache()
