"""The parity tests' error measure (tests/gpu_util.py norm_error) on cases
whose answer is fixed by IEEE rounding, on the CPU.

A result in float16's subnormal range (below 2^-14) rounded once to nearest
errs by up to half the subnormal spacing 2^-24, an absolute 2^-25 that can be
more than 2^-11 of the result; the measure subtracts that floor, so a
correctly rounded subnormal passes while an error a whole subnormal step
larger does not.
"""
import numpy as np

from tests.gpu_util import SUBNORMAL_FLOOR, TOL, norm_error


def test_float16_subnormal_rounding_is_within_the_bound():
    # one product x*w of 2.124e-5 (the value a random-grid case produced),
    # with no bias: the denominator is |x*w| itself
    y_ref = np.array([2.124177262885496e-05])
    y_gpu = y_ref.astype(np.float16).astype(np.float64)  # one round-to-nearest-even
    scale = np.abs(y_ref)
    assert norm_error(y_gpu, y_ref, scale, np.zeros(1)) > TOL["f16"]  # relative bound alone
    assert norm_error(y_gpu, y_ref, scale, np.zeros(1), dtype="f16") <= TOL["f16"]


def test_a_whole_subnormal_step_more_is_still_caught():
    y_ref = np.array([2.124177262885496e-05])
    y_rn = y_ref.astype(np.float16).astype(np.float64)
    y_gpu = y_rn + np.sign(y_rn - y_ref) * 2.0 ** -24  # one more subnormal step, away from y_ref
    assert norm_error(y_gpu, y_ref, np.abs(y_ref), np.zeros(1), dtype="f16") > TOL["f16"]


def test_floor_is_half_the_subnormal_spacing():
    # the smallest positive subnormal of each type, halved
    assert SUBNORMAL_FLOOR["f16"] == float(np.finfo(np.float16).smallest_subnormal) / 2
    assert SUBNORMAL_FLOOR["f32"] == float(np.finfo(np.float32).smallest_subnormal) / 2
    assert SUBNORMAL_FLOOR["bf16"] == 2.0 ** -133 / 2  # bfloat16: float32's exponent, 7 fraction bits


def test_zero_denominator_still_needs_an_exact_zero():
    assert norm_error(np.array([2.0 ** -30]), np.zeros(1), np.zeros(1), np.zeros(1), dtype="f16") == float("inf")
