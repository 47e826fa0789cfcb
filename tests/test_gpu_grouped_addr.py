"""Grouped route with the output at a device address whose low 32-bit word has
bit 31 set.

The grouped kernel forms the output's buffer resource from the address words
read from lane 0; a low word taken as a signed value was once sign-extended
into the high word there, which moved the resource's base. These cases place
y inside a larger buffer so that its address has that bit, for the segment-pair
instance (width stride 2, 8 channels per group, whole 128-byte rows) and for
the general one (odd output width), and compare every output with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import convt_forward_amd as C
import workloads
from tests.gpu_util import TOL, bias_abs_full, norm_error, oracle_full, say, to_device, to_host64

# (name, x shape, W shape, stride, padding, dilation, output_padding, groups)
CASES = [
    ("segment_pairs", (2, 32, 16, 32), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4),
    ("general", (2, 32, 7, 9), (32, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 4),
]


def _offset_with_bit31(addr: int, nbytes: int) -> int:
    """An offset at which [addr + off, + nbytes) has bit 31 of the low address
    word set throughout: 0, or the one that moves the low word to 2^31 (it
    keeps addr's alignment up to 2^31). At most 2^31 + nbytes."""
    lo = addr & 0xFFFFFFFF
    if lo >= 0x80000000 and lo + nbytes <= 0xFFFFFFFF:
        return 0
    return (0x80000000 - lo) % (1 << 32)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_output_address_with_bit31(case, dtype):
    import torch
    name, xs, wsh, s, p, d, op, g = case
    tens = workloads.make_tensors(xs, wsh, wsh[1] * g, True, dtype, "uniform", "uniform", "uniform", 71)
    pl = C.get_plan(xs, wsh, s, p, d, op, g, True, dtype)
    assert pl.route == "grouped", pl.route
    out_shape = tuple(pl.out_shape)
    nbytes = int(np.prod(out_shape)) * 2
    base = torch.empty((1 << 31) + 2 * nbytes + 512, dtype=torch.uint8, device="cuda")
    off = _offset_with_bit31(base.data_ptr(), nbytes)
    assert off + nbytes <= base.numel()
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    y = base[off:off + nbytes].view(tdt).view(out_shape)
    assert (y.data_ptr() & 0x80000000) and ((y.data_ptr() + nbytes - 1) & 0x80000000)
    say(f"[gpu] grouped {name} {dtype}: y at {y.data_ptr():#x}")
    x = to_device(tens.x_dev, dtype)
    w = to_device(tens.w_dev, dtype)
    b = to_device(tens.bias_dev, dtype)
    pl.forward(x, w, b, y=y)
    torch.cuda.synchronize()
    ref, sc = oracle_full(tens, dict(stride=s, padding=p, dilation=d, output_padding=op, groups=g))
    e = norm_error(to_host64(y), ref, sc, bias_abs_full(tens, ref.shape), dtype=dtype)
    del base
    assert e <= TOL[dtype], f"{name} {dtype}: error {e}"
