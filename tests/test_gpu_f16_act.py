"""GPU parity of the float16 element type and of the fused activation
(through the C ABI, against the oracle).

float16 (IEEE half; the huggingface page's shader-f16 variants): inputs,
weights, bias and output in half, float32 accumulation, one rounding; bound
1e-3 on the normalised error (tests/gpu_util.py), exact on integer data
(equal to the oracle rounded once to half).

Activation (the AWS Neuron page's activation_fn; the set and its placement,
after the bias and before the rounding, are the reading in include/convt.h):
the error denominator becomes L_f * (scale + |bias|) + |f(y)|, L_f the
activation's Lipschitz constant, so that the pre-activation error carried
through f and the rounding of f's value are both allowed for.
"""
import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests.gpu_util import TOL, check_full, say, to_device, to_host64, norm_error

pytestmark = pytest.mark.gpu

ROUTES = ["auto", "naive", "direct", "phase_gemm", "phase_gemm_packed", "phase_gemm_allphase", "grouped"]

CASES = [
    # name, x shape, w shape, stride, pad, dil, op, groups
    ("c1_like", (2, 4, 8, 8), (4, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1),
    ("c2_like", (2, 40, 300), (40, 24, 8), (4,), (2,), (1,), (0,), 1),
    ("c3_like", (2, 72, 9, 13), (72, 136, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1),
    ("c4a_like", (2, 32, 7, 9), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4),
    ("c4b_like", (2, 40, 11, 13), (40, 40, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1),
    ("c5_like", (1, 40, 3, 5, 7), (40, 24, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1),
]


def prm_of(c, act="none"):
    return dict(stride=c[3], padding=c[4], dilation=c[5], output_padding=c[6], groups=c[7],
                activation=act)


def serves(c, dt, route, act="none"):
    try:
        C.get_plan(c[1], c[2], c[3], c[4], c[5], c[6], c[7], True, dt, route, activation=act)
        return True
    except C.ConvtError as e:
        assert e.status == 2
        return False


def rne_f16(v):
    return v.astype(np.float32).astype(np.float16).astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("route", ROUTES)
def test_float16_every_route(case, route):
    if not serves(case, "f16", route):
        pytest.skip(f"route {route} does not serve this problem")
    tens = workloads.make_tensors(case[1], case[2], case[2][1] * case[7], True, "f16", "uniform",
                                  "uniform", "uniform", 60)
    check_full(tens, prm_of(case), route=route, tag=f"f16 {case[0]}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("route", ROUTES)
def test_float16_integer_exact(case, route):
    import torch
    if not serves(case, "f16", route):
        pytest.skip(f"route {route} does not serve this problem")
    tens = workloads.make_tensors(case[1], case[2], case[2][1] * case[7], True, "f16", "int(4)",
                                  "int(4)", "int(4)", 61)
    say(f"[gpu] f16 integer {case[0]} route={route}")
    pl = C.get_plan(case[1], case[2], case[3], case[4], case[5], case[6], case[7], True, "f16",
                    route)
    y = pl.forward(to_device(tens.x_dev, "f16"), to_device(tens.w_dev, "f16"),
                   to_device(tens.bias_dev, "f16"))
    torch.cuda.synchronize()
    ref, _ = oracle.forward(tens.x, tens.w, tens.bias, case[3], case[4], case[5], case[6],
                            case[7], with_scale=False)
    bad = np.argwhere(to_host64(y) != rne_f16(ref))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("case", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_float16_backward_data(case):
    import torch
    prm = prm_of(case)
    ys = oracle.out_shape(case[1], case[2], case[3], case[4], case[5], case[6], case[7])
    t = workloads.make_tensors(ys, case[2], 0, False, "f16", "uniform", "uniform", "uniform", 62)
    for route in ["auto", "naive", "phase_gemm", "direct"]:
        try:
            pl = C.get_plan(case[1], case[2], case[3], case[4], case[5], case[6], case[7], False,
                            "f16", "auto", route)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        say(f"[gpu] f16 backward {case[0]} route={pl.route_bwd}")
        dx = pl.backward_data(to_device(t.x_dev, "f16"), to_device(t.w_dev, "f16"))
        torch.cuda.synchronize()
        ref, sc = oracle.backward_data(t.x, t.w, case[1], case[3], case[4], case[5], case[6],
                                       case[7])
        e = norm_error(to_host64(dx), ref, sc, np.zeros_like(sc), dtype="f16")
        assert e <= TOL["f16"], f"backward {route}: {e}"


ACTS = ["relu", "sigmoid", "tanh", "silu", "gelu"]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_activation_every_route(case, act, dt):
    # normal(1) data spreads the pre-activation values over every regime of f
    tens = workloads.make_tensors(case[1], case[2], case[2][1] * case[7], True, dt, "normal(1)",
                                  "normal(0.5)", "normal(1)", 63)
    for route in ROUTES:
        if serves(case, dt, route, act):
            check_full(tens, prm_of(case, act), route=route, tag=f"{act} {dt} {case[0]}")


def test_activation_on_the_fill_route():
    """No input channels: every output is f(bias)."""
    import torch
    for act in ACTS:
        for dt in ["f32", "bf16", "f16"]:
            tens = workloads.make_tensors((2, 0, 5, 6), (0, 3, 3, 3), 3, True, dt, "uniform",
                                          "uniform", "normal(2)", 64)
            pl = C.get_plan((2, 0, 5, 6), (0, 3, 3, 3), 2, 1, 1, 0, 1, True, dt, activation=act)
            assert pl.route == "fill"
            say(f"[gpu] fill {act} {dt}")
            x = to_device(np.zeros((2, 0, 5, 6), np.float32 if dt == "f32" else np.uint16), dt)
            w = to_device(np.zeros((0, 3, 3, 3), np.float32 if dt == "f32" else np.uint16), dt)
            y = pl.forward(x, w, to_device(tens.bias_dev, dt))
            torch.cuda.synchronize()
            ref = oracle.activation(C.ACTIVATIONS[act], tens.bias.astype(np.float64))
            got = to_host64(y)
            den = np.abs(ref) + 1e-30
            err = np.max(np.abs(got - ref[None, :, None, None]) / den[None, :, None, None])
            assert err <= TOL[dt], (act, dt, err)
