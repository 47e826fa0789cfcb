"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case prints what it runs before touching the GPU. Tolerances and the
error measure are described in tests/gpu_util.py.
"""
import itertools

import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests import oracle_pins
from tests.gpu_util import (TOL, bias_abs_full, check_full, check_sampled, norm_error,
                            oracle_full, params_of, run_gpu, sample_points, say, to_device,
                            to_host64)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# The five workloads at their full sizes, in the launch configuration the
# benchmark times (automatic route).
# ---------------------------------------------------------------------------
FULL_ORACLE = ["c1", "c2", "c3", "c4a", "c4b", "c5"]


# every output of every workload against the full oracle (the threaded
# double-precision scatter takes seconds per workload on the host cores)
@pytest.mark.parametrize("name", FULL_ORACLE)
def test_workload_full_size_all_outputs(name):
    wl = workloads.get(name)
    tens = workloads.workload_tensors(wl)
    check_full(tens, params_of(wl), tag=wl.name)


# ---------------------------------------------------------------------------
# Reduced versions of the workloads (same attributes) whose full outputs the
# oracle computes in seconds; chosen to span several tiles with ragged tails
# in channels and positions.
# ---------------------------------------------------------------------------
REDUCED = [
    # name, x shape, w shape, stride, pad, dil, op, groups, dtype, dist
    ("c1_like_f32", (2, 4, 8, 8), (4, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1, "f32"),
    ("c2_like_f32", (2, 40, 300), (40, 24, 8), (4,), (2,), (1,), (0,), 1, "f32"),
    ("c2_like_f32_wide", (1, 128, 150), (128, 64, 8), (4,), (2,), (1,), (0,), 1, "f32"),
    ("c3_like_bf16", (2, 72, 9, 13), (72, 136, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, "bf16"),
    ("c3_like_f32", (2, 40, 9, 13), (40, 70, 4, 4), (2, 2), (1, 1), (1, 1), (1, 0), 1, "f32"),
    ("c4a_like_bf16", (2, 32, 7, 9), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4, "bf16"),
    ("c4b_like_bf16", (2, 40, 11, 13), (40, 40, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1, "bf16"),
    ("c5_like_bf16", (1, 40, 3, 5, 7), (40, 24, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1,
     "bf16"),
]


def reduced_tensors(case, seed, dist="uniform", bias=True):
    name, xs, ws, s, p, d, op, g, dt = case
    tens = workloads.make_tensors(xs, ws, ws[1] * g, bias, dt, dist, dist, dist, seed)
    prm = dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g)
    return tens, prm


@pytest.mark.parametrize("case", REDUCED, ids=[c[0] for c in REDUCED])
def test_reduced_workloads(case):
    tens, prm = reduced_tensors(case, seed=7)
    check_full(tens, prm, tag=case[0])


@pytest.mark.parametrize("case", REDUCED, ids=[c[0] for c in REDUCED])
@pytest.mark.parametrize("route", ["naive", "direct", "phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "grouped"])
def test_reduced_workloads_every_route(case, route):
    tens, prm = reduced_tensors(case, seed=8)
    try:
        C.get_plan(tens.x.shape, tens.w.shape, prm["stride"], prm["padding"], prm["dilation"],
                   prm["output_padding"], prm["groups"], True, tens.dtype, route)
    except C.ConvtError as e:
        assert e.status == 2
        pytest.skip(f"route {route} does not serve this problem")
    check_full(tens, prm, route=route, tag=f"{case[0]}/{route}")


# ---------------------------------------------------------------------------
# Integer data: every partial sum is an integer below 2^24, so float32
# accumulation is exact in any order. float32 outputs must equal the oracle
# bit for bit; bfloat16 outputs must equal the oracle rounded once to
# bfloat16 (round to nearest even).
# ---------------------------------------------------------------------------
def rne_bf16(v: np.ndarray) -> np.ndarray:
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v.astype(np.float32))).astype(
        np.float64)


@pytest.mark.parametrize("case", REDUCED, ids=[c[0] for c in REDUCED])
@pytest.mark.parametrize("route", ["auto", "naive", "direct", "phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "grouped"])
def test_integer_inputs_exact(case, route):
    tens, prm = reduced_tensors(case, seed=9, dist="int(4)")
    try:
        C.get_plan(tens.x.shape, tens.w.shape, prm["stride"], prm["padding"], prm["dilation"],
                   prm["output_padding"], prm["groups"], True, tens.dtype, route)
    except C.ConvtError as e:
        assert e.status == 2
        pytest.skip(f"route {route} does not serve this problem")
    say(f"[gpu] integer {case[0]} route={route}")
    y, _ = run_gpu(tens, prm, route)
    ref, _ = oracle_full(tens, prm)
    assert np.all(ref == np.round(ref))
    expect = ref if tens.dtype == "f32" else rne_bf16(ref)
    bad = np.argwhere(y != expect)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}: {y[tuple(bad[0])]} vs {expect[tuple(bad[0])]}"


def test_integer_inputs_exact_full_c3_sampled():
    wl = workloads.get("c3")
    tens = workloads.make_tensors(wl.x_shape, wl.w_shape, wl.c_out, True, "bf16", "int(4)",
                                  "int(4)", "int(4)", 33)
    prm = params_of(wl)
    say("[gpu] integer c3 full size")
    y, _ = run_gpu(tens, prm)
    pts = sample_points(y.shape, np.random.default_rng(101))
    _, got, yv = check_sampled(y, tens, prm, pts)
    assert np.array_equal(got, rne_bf16(yv))


# ---------------------------------------------------------------------------
# Seeded random grid over ranks, strides, kernels, dilations, paddings
# (including pads beyond d*(k-1)), output paddings, groups and dtypes, on
# every route that serves each problem.
# ---------------------------------------------------------------------------
def grid_cases(n, seed, asym=False):
    rng = np.random.default_rng(seed)
    out = []
    for prm in oracle_pins.random_grid(rng, n, asym=asym):
        scale_c = int(rng.choice([1, 1, 4, 12]))
        prm = dict(prm)
        prm["Ci"] *= scale_c
        prm["Cog"] = int(prm["Cog"] * int(rng.choice([1, 3, 20])))
        prm["dtype"] = str(rng.choice(["f32", "bf16"]))
        prm["seed"] = int(rng.integers(0, 2**31))
        out.append(prm)
    return out


GRID = grid_cases(60, 2024)
# the same with different low and high padding on about half the cases
GRID_ASYM = grid_cases(40, 2025, asym=True)


def grid_params(prm):
    pad = tuple(prm["p"]) if prm["p"] == prm["ph"] else tuple(zip(prm["p"], prm["ph"]))
    return dict(stride=tuple(prm["s"]), padding=pad, dilation=tuple(prm["d"]),
                output_padding=tuple(prm["op"]), groups=prm["groups"])


@pytest.mark.parametrize("idx", range(len(GRID)))
def test_random_grid_all_routes(idx):
    run_grid_case(GRID[idx], f"grid[{idx}]")


@pytest.mark.parametrize("idx", range(len(GRID_ASYM)))
def test_random_grid_asymmetric_padding_all_routes(idx):
    run_grid_case(GRID_ASYM[idx], f"grid_asym[{idx}]")


def run_grid_case(prm, tag):
    xs = (prm["B"], prm["Ci"]) + tuple(prm["I"])
    ws = (prm["Ci"], prm["Cog"]) + tuple(prm["k"])
    params = grid_params(prm)
    has_bias = bool(prm["seed"] % 2)
    tens = workloads.make_tensors(xs, ws, prm["Cog"] * prm["groups"], has_bias, prm["dtype"],
                                  "normal(1)", "normal(1)", "normal(1)", prm["seed"])
    for route in ["auto", "naive", "direct", "phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "grouped"]:
        try:
            C.get_plan(xs, ws, params["stride"], params["padding"], params["dilation"],
                       params["output_padding"], params["groups"], has_bias, prm["dtype"], route)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        check_full(tens, params, route=route, tag=tag)


GROUPED = [
    # x shape, w shape, stride, pad, dil, op, groups
    ((2, 16, 9), (16, 5, 4), (2,), (1,), (1,), (0,), 2),
    ((1, 48, 6, 7), (48, 16, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 3),
    ((2, 64, 5, 6), (64, 3, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 8),
    ((1, 16, 7, 10), (16, 8, 5, 3), (3, 2), (2, 1), (1, 2), (2, 1), 2),
    ((1, 24, 3, 4, 5), (24, 4, 3, 2, 2), (2, 1, 2), (1, 0, 1), (1, 1, 1), (1, 0, 0), 1),
    ((2, 32, 8, 8), (32, 8, 4, 4), (1, 1), (1, 1), (1, 1), (0, 0), 4),
    ((1, 16, 4, 33), (16, 16, 2, 4), (4, 2), (0, 1), (1, 1), (3, 1), 2),
    # input rows of whole 16-byte chunks (the chunked halo gather): borders,
    # chunks left of the row (dilation 5), width strides 1..4, 3-D
    ((2, 16, 5, 16), (16, 4, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 2),
    ((1, 32, 3, 24), (32, 8, 4, 5), (1, 3), (2, 3), (1, 1), (0, 2), 2),
    ((1, 64, 4, 8, 16), (64, 2, 2, 3, 4), (2, 2, 4), (0, 1, 1), (1, 1, 1), (0, 0, 3), 8),
    ((1, 16, 6, 16), (16, 8, 3, 3), (1, 1), (0, 0), (5, 5), (0, 0), 2),
    ((3, 32, 9, 40), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4),
]


@pytest.mark.parametrize("idx", range(len(GROUPED)))
def test_grouped_route_cases(idx):
    xs, ws, s, p, d, op, g = GROUPED[idx]
    params = dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g)
    tens = workloads.make_tensors(xs, ws, ws[1] * g, True, "bf16", "uniform", "uniform", "uniform",
                                  500 + idx)
    for route in ["grouped", "auto", "phase_gemm"]:
        check_full(tens, params, route=route, tag=f"grouped[{idx}]")


# ---------------------------------------------------------------------------
# Different low and high padding per axis (the AWS Neuron conv3d_transpose
# page's padding pairs): workload-like shapes on every route, with pads that
# trim only one end, pads beyond d*(k-1) and zero pads next to large ones.
# ---------------------------------------------------------------------------
ASYM = [
    # name, x shape, w shape, stride, (lo, hi) pads, dil, op, groups, dtype
    ("c1_like_f32", (2, 4, 8, 8), (4, 8, 3, 3), (2, 2), ((1, 0), (0, 2)), (1, 1), (1, 1), 1, "f32"),
    ("c2_like_f32", (2, 40, 300), (40, 24, 8), (4,), ((3, 1),), (1,), (0,), 1, "f32"),
    ("c3_like_bf16", (2, 72, 9, 13), (72, 136, 4, 4), (2, 2), ((0, 2), (2, 1)), (1, 1), (0, 0), 1,
     "bf16"),
    ("c4a_like_bf16", (2, 32, 7, 9), (32, 8, 4, 4), (2, 2), ((2, 0), (0, 1)), (1, 1), (0, 0), 4,
     "bf16"),
    ("c4b_like_bf16", (2, 40, 11, 13), (40, 40, 3, 3), (1, 1), ((0, 4), (3, 1)), (2, 2), (0, 0), 1,
     "bf16"),
    ("c5_like_bf16", (1, 40, 3, 5, 7), (40, 24, 4, 4, 4), (2, 2, 2), ((1, 2), (0, 1), (2, 0)),
     (1, 1, 1), (0, 0, 0), 1, "bf16"),
    ("beyond_dk_f32", (1, 16, 6, 7), (16, 8, 3, 3), (2, 2), ((4, 0), (0, 5)), (1, 1), (1, 0), 1,
     "f32"),
    ("grouped_chunks_bf16", (2, 16, 5, 16), (16, 4, 3, 3), (2, 2), ((0, 2), (2, 0)), (1, 1), (1, 1),
     2, "bf16"),
]


@pytest.mark.parametrize("case", ASYM, ids=[c[0] for c in ASYM])
@pytest.mark.parametrize("route", ["auto", "naive", "direct", "phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "grouped"])
def test_asymmetric_padding_every_route(case, route):
    name, xs, ws, s, p, d, op, g, dt = case
    prm = dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g)
    for dist, seed in (("uniform", 40), ("int(4)", 41)):
        tens = workloads.make_tensors(xs, ws, ws[1] * g, True, dt, dist, dist, dist, seed)
        try:
            C.get_plan(xs, ws, s, p, d, op, g, True, dt, route)
        except C.ConvtError as e:
            assert e.status == 2
            pytest.skip(f"route {route} does not serve this problem")
        if dist == "uniform":
            check_full(tens, prm, route=route, tag=f"asym {name}/{route}")
            continue
        say(f"[gpu] integer asym {name} route={route}")
        y, _ = run_gpu(tens, prm, route)
        ref, _ = oracle_full(tens, prm)
        expect = ref if dt == "f32" else rne_bf16(ref)
        bad = np.argwhere(y != expect)
        assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def test_empty_batch():
    say("[gpu] empty batch")
    tens = workloads.make_tensors((0, 3, 5), (3, 2, 3), 2, True, "f32", "uniform", "uniform",
                                  "uniform", 1)
    y, pl = run_gpu(tens, dict(stride=(2,), padding=(1,), dilation=(1,), output_padding=(0,),
                               groups=1))
    assert pl.route == "none" and y.shape == (0, 2, 9)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_input_channels_is_bias(dtype):
    say(f"[gpu] C_in = 0 ({dtype})")
    tens = workloads.make_tensors((2, 0, 5), (0, 3, 3), 3, True, dtype, "uniform", "uniform",
                                  "uniform", 2)
    prm = dict(stride=(2,), padding=(1,), dilation=(1,), output_padding=(1,), groups=1)
    y, pl = run_gpu(tens, prm)
    assert pl.route == "fill"
    assert np.array_equal(y, np.broadcast_to(tens.bias.reshape(1, 3, 1), y.shape))


def test_empty_input_axis_is_bias():
    say("[gpu] empty input axis")
    tens = workloads.make_tensors((2, 3, 0), (3, 2, 3), 2, True, "f32", "uniform", "uniform",
                                  "uniform", 3)
    prm = dict(stride=(1,), padding=(0,), dilation=(1,), output_padding=(0,), groups=1)
    y, pl = run_gpu(tens, prm)
    assert y.shape == (2, 2, 2) and pl.route == "fill"
    assert np.array_equal(y, np.broadcast_to(tens.bias.reshape(1, 2, 1), y.shape))


@pytest.mark.parametrize("route", ["auto", "phase_gemm", "naive", "direct"])
def test_phases_without_taps(route):
    # kernel 2, stride 4: residues 2 and 3 receive no products, only the bias
    tens = workloads.make_tensors((2, 20, 9), (20, 70, 2), 70, True, "f32", "uniform", "uniform",
                                  "uniform", 4)
    prm = dict(stride=(4,), padding=(0,), dilation=(1,), output_padding=(3,), groups=1)
    y, _, _ = check_full(tens, prm, route=route, tag="empty phases")
    assert np.array_equal(y[:, :, 2::4], np.broadcast_to(tens.bias.reshape(1, -1, 1), y[:, :, 2::4].shape))


def test_large_stride_uses_naive():
    tens = workloads.make_tensors((1, 3, 4), (3, 2, 3), 2, True, "f32", "uniform", "uniform",
                                  "uniform", 5)
    prm = dict(stride=(19,), padding=(1,), dilation=(1,), output_padding=(5,), groups=1)
    _, _, pl = check_full(tens, prm, tag="stride 19")
    assert pl.route in ("naive", "direct")


def test_deterministic_and_stream_independent():
    import torch
    wl = workloads.get("c3")
    tens = workloads.workload_tensors(wl)
    prm = params_of(wl)
    say("[gpu] c3 determinism / side stream")
    y1, _ = run_gpu(tens, prm)
    s = torch.cuda.Stream()
    y2, _ = run_gpu(tens, prm, stream=s.cuda_stream)
    assert np.array_equal(y1, y2)


# A call on a side stream that lets the binding allocate y and the workspace:
# those allocations come from torch's current stream, and are freed (the
# workspace) when the call returns while the kernels on the side stream may
# still run. The binding records them on the side stream; without that, the
# buffer allocated and filled on the current stream right after the call
# could take the workspace's memory under the running GEMM.
@pytest.mark.parametrize("as_handle", [False, True])
def test_side_stream_allocations_not_reused(as_handle):
    import torch
    wl = workloads.get("c3")
    tens = workloads.workload_tensors(wl)
    prm = params_of(wl)
    say(f"[gpu] c3 side stream, binding-allocated buffers (handle={as_handle})")
    y_ref, pl = run_gpu(tens, prm)
    x = to_device(tens.x_dev, "bf16")
    w = to_device(tens.w_dev, "bf16")
    b = to_device(tens.bias_dev, "bf16")
    side = torch.cuda.Stream()
    # the side stream starts behind a long busy kernel, so that the
    # convolution is still queued when the host returns
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        busy = torch.randn(4096, 4096, device="cuda")
        for _ in range(8):
            busy = busy @ busy
            busy /= busy.norm()
    y = pl.forward(x, w, b, stream=side.cuda_stream if as_handle else side)
    junk = []
    for _ in range(4):
        t = torch.empty(pl.workspace_bytes, dtype=torch.uint8, device="cuda")
        t.fill_(0x5a)
        junk.append(t)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y), y_ref)
    del busy, junk


# convt_forward runs the two-byte GEMM's weight reorder and input copy as one
# launch; the split API runs them as two. Both must give the same bytes, on
# planes of whole 16-byte rows (the copy through LDS) and others.
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("hw", [(11, 13), (8, 16)])
def test_prepared_split_matches_forward(dt, hw):
    import torch
    xs = (2, 40) + hw
    tens = workloads.make_tensors(xs, (40, 40, 3, 3), 40, True, dt, "uniform",
                                  "uniform", "uniform", 6)
    prm = dict(stride=(1, 1), padding=(2, 2), dilation=(2, 2), output_padding=(0, 0), groups=1)
    say(f"[gpu] prepare_weights + forward_prepared {dt} {hw}")
    y_ref, pl = run_gpu(tens, prm, route="phase_gemm_packed")
    assert pl.route == "phase_gemm_packed"
    x = to_device(tens.x_dev, dt)
    w = to_device(tens.w_dev, dt)
    b = to_device(tens.bias_dev, dt)
    ws = pl.new_workspace(x.device)
    y = pl.new_output(x.device)
    st = torch.cuda.current_stream().cuda_stream
    pl.prepare_weights_ptr(w.data_ptr(), ws.data_ptr(), st)
    pl.forward_prepared_ptr(x.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr(), ws.data_ptr(), st)
    # the prepared weights serve a second input too
    x2 = to_device(workloads.make_tensors(xs, (40, 40, 3, 3), 40, True, dt,
                                          "uniform", "uniform", "uniform", 7).x_dev, dt)
    y2 = pl.new_output(x.device)
    pl.forward_prepared_ptr(x2.data_ptr(), w.data_ptr(), b.data_ptr(), y2.data_ptr(), ws.data_ptr(), st)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y), y_ref)
    y2_ref = pl.forward(x2, w, b)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y2), to_host64(y2_ref))


# The same split on the GEMM that reads x in place (even rows, more than 64
# output channels): convt_forward is the reorder then that kernel.
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prepared_split_matches_forward_in_place(dt):
    import torch
    xs, ws = (2, 40, 10, 16), (40, 96, 4, 4)
    tens = workloads.make_tensors(xs, ws, 96, True, dt, "uniform", "uniform", "uniform", 16)
    prm = dict(stride=(2, 2), padding=(1, 1), dilation=(1, 1), output_padding=(0, 0), groups=1)
    say(f"[gpu] prepare_weights + forward_prepared in place {dt}")
    y_ref, pl = run_gpu(tens, prm, "phase_gemm")
    assert pl.route == "phase_gemm"
    x = to_device(tens.x_dev, dt)
    w = to_device(tens.w_dev, dt)
    b = to_device(tens.bias_dev, dt)
    ws_t = pl.new_workspace(x.device)
    y = pl.new_output(x.device)
    st = torch.cuda.current_stream().cuda_stream
    pl.prepare_weights_ptr(w.data_ptr(), ws_t.data_ptr(), st)
    pl.forward_prepared_ptr(x.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr(), ws_t.data_ptr(), st)
    torch.cuda.synchronize()
    assert np.array_equal(to_host64(y), y_ref)


# ---------------------------------------------------------------------------
# Maximum sizes: planes of 2^25 - 2^26 positions, channel slices of 1 GiB
# (the raw buffer resources' 32-bit byte offsets at half their range), on
# every route that serves them, checked on sampled outputs.
# ---------------------------------------------------------------------------
# (the 2-D cases once wrote zeros over real outputs: tile rows past C_out
# had their channel offset wrap the 32-bit range)
LARGE = [
    ("1d_2^24", (1, 16, 1 << 24), (16, 8, 4), (2,), (1,), (1,), (0,), 1, "bf16"),
    ("2d_4096^2", (1, 8, 4096, 4096), (8, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1, "bf16"),
    ("2d_2896^2_f32", (1, 8, 2896, 2896), (8, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1, "f32"),
]


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_large_planes_sampled(case):
    import torch
    name, xs, ws, s, p, d, op, g, dt = case
    prm = dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g)
    tens = workloads.make_tensors(xs, ws, ws[1] * g, True, dt, "uniform", "uniform",
                                  "uniform", 77)
    x = to_device(tens.x_dev, dt)
    w = to_device(tens.w_dev, dt)
    b = to_device(tens.bias_dev, dt)
    pts = None
    for route in ["auto", "phase_gemm", "grouped", "direct", "naive"]:
        try:
            pl = C.get_plan(xs, ws, s, p, d, op, g, True, dt, route)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        say(f"[gpu] large {name} route={pl.route}")
        y = pl.forward(x, w, b)
        torch.cuda.synchronize()
        if pts is None:
            rng = np.random.default_rng(103)
            pts = np.stack([rng.integers(0, v, 20000) for v in y.shape], axis=1).astype(np.int64)
            # the last outputs of the plane (the far end of the offsets)
            last = np.array(np.unravel_index(np.arange(y[0, 0].numel() - 64, y[0, 0].numel()),
                                             tuple(y.shape[2:]))).T
            tail = np.concatenate([np.tile([[0, y.shape[1] - 1]], (64, 1)), last], axis=1)
            pts = np.concatenate([pts, tail.astype(np.int64)])
            yv, sv = oracle.points(tens.x, tens.w, tens.bias, pts, s, p, d, op, g)
            babs = np.abs(tens.bias[pts[:, 1]].astype(np.float64))
        got = to_host64(y[tuple(torch.from_numpy(pts.T).to(y.device))])
        e = norm_error(got, yv, sv, babs, dtype=dt)
        say(f"[gpu]   -> {len(pts)} points, max normalised error {e:.3e}")
        assert e <= TOL[dt], f"{route}: {e}"
        del y
        torch.cuda.empty_cache()
