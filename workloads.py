"""Seeded synthetic inputs for the ConvTranspose forward workloads.

This module is shared by the tests, the benchmark and the smoke check. It
holds the workload table (shapes, attributes, value distributions, seeds) and
the random-number draws, and nothing of the operation's own arithmetic: no
output-size formula, no phase plan, no products or sums. Both the HIP path and
the CPU oracle consume the exact host buffers made here.

Recipe (the same for every workload):
  * numpy ``default_rng(seed)`` (PCG64), values drawn in float64 in the order
    x, W, bias, each as one flat draw of the tensor's element count;
  * "uniform" is U[-1, 1), "normal(s)" is N(0, s^2) (s is a standard deviation);
  * cast to float32; for bfloat16 workloads the float32 values are then rounded
    to bfloat16 (round to nearest, ties to even, on the float32 bit pattern),
    so the float32 copy holds exactly the bfloat16 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Workload table. Shapes follow the layouts the pages use: x is
# [B, C_in, spatial...], W is [C_in, C_out/groups, k...], bias is [C_out].
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    x_shape: Tuple[int, ...]
    w_shape: Tuple[int, ...]
    stride: Tuple[int, ...]
    padding: Tuple[int, ...]
    dilation: Tuple[int, ...]
    output_padding: Tuple[int, ...]
    groups: int
    has_bias: bool
    dtype: str  # "f32", "bf16" or "f16"
    x_dist: str
    w_dist: str
    b_dist: str
    seed: int

    @property
    def ndim(self) -> int:
        return len(self.x_shape) - 2

    @property
    def c_out(self) -> int:
        return self.w_shape[1] * self.groups


WORKLOADS = {
    "c1_2d_f32_small": Workload(
        "c1_2d_f32_small",
        "ConvTranspose2d fp32 x[1,4,8,8] W[4,8,3,3] stride 2 pad 1 output_padding 1 bias[8]",
        (1, 4, 8, 8), (4, 8, 3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 1, True, "f32",
        "uniform", "uniform", "uniform", 1),
    "c2_1d_f32_upsampler": Workload(
        "c2_1d_f32_upsampler",
        "ConvTranspose1d fp32 x[16,128,1024] W[128,64,8] stride 4 pad 2 bias[64] (audio-decoder upsampler)",
        (16, 128, 1024), (128, 64, 8), (4,), (2,), (1,), (0,), 1, True, "f32",
        "normal(1)", "normal(1)", "normal(1)", 2),
    "c3_2d_bf16_generator": Workload(
        "c3_2d_bf16_generator",
        "ConvTranspose2d bf16 x[64,512,16,16] W[512,256,4,4] stride 2 pad 1 bias[256] (generator upsampling)",
        (64, 512, 16, 16), (512, 256, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 1, True, "bf16",
        "normal(1)", "normal(0.02)", "normal(0.02)", 3),
    "c4a_2d_bf16_grouped": Workload(
        "c4a_2d_bf16_grouped",
        "Grouped ConvTranspose2d bf16 x[32,256,32,32] W[256,8,4,4] groups 32 stride 2 pad 1 bias[256]",
        (32, 256, 32, 32), (256, 8, 4, 4), (2, 2), (1, 1), (1, 1), (0, 0), 32, True, "bf16",
        "uniform", "uniform", "uniform", 4),
    "c4b_2d_bf16_dilated": Workload(
        "c4b_2d_bf16_dilated",
        "ConvTranspose2d bf16 x[32,128,64,64] W[128,128,3,3] stride 1 pad 2 dilation 2 bias[128]",
        (32, 128, 64, 64), (128, 128, 3, 3), (1, 1), (2, 2), (2, 2), (0, 0), 1, True, "bf16",
        "uniform", "uniform", "uniform", 6),
    "c5_3d_bf16_video": Workload(
        "c5_3d_bf16_video",
        "ConvTranspose3d bf16 x[2,256,8,32,32] W[256,128,4,4,4] stride 2 pad 1 bias[128] (video-decoder upsample)",
        (2, 256, 8, 32, 32), (256, 128, 4, 4, 4), (2, 2, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, True,
        "bf16", "normal(1)", "normal(0.02)", "normal(0.02)", 5),
}

# Short aliases used on command lines.
ALIASES = {
    "c1": "c1_2d_f32_small",
    "c2": "c2_1d_f32_upsampler",
    "c3": "c3_2d_bf16_generator",
    "c4a": "c4a_2d_bf16_grouped",
    "c4b": "c4b_2d_bf16_dilated",
    "c5": "c5_3d_bf16_video",
}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


# ---------------------------------------------------------------------------
# Random draws
# ---------------------------------------------------------------------------


def _draw(rng: np.random.Generator, dist: str, n: int) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=n)
    if dist.startswith("normal(") and dist.endswith(")"):
        sd = float(dist[len("normal("):-1])
        return rng.normal(0.0, sd, size=n)
    if dist.startswith("int(") and dist.endswith(")"):
        # integers drawn uniformly from [-m, m]
        m = int(dist[len("int("):-1])
        return rng.integers(-m, m + 1, size=n).astype(np.float64)
    raise ValueError(f"unknown distribution {dist!r}")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensors:
    """Host buffers of one problem instance.

    ``x``, ``w``, ``bias`` are float32 arrays holding the exact values (for
    bfloat16 / float16 problems, exactly representable in that type). ``x_dev``
    etc. are the arrays in the device dtype, ready to be copied to the GPU:
    float32 arrays, or uint16 bit patterns of bfloat16 or IEEE half.
    """
    dtype: str
    x: np.ndarray
    w: np.ndarray
    bias: Optional[np.ndarray]
    x_dev: np.ndarray = field(repr=False, default=None)
    w_dev: np.ndarray = field(repr=False, default=None)
    bias_dev: Optional[np.ndarray] = field(repr=False, default=None)


def make_tensors(x_shape: Sequence[int], w_shape: Sequence[int], c_out: int, has_bias: bool,
                 dtype: str, x_dist: str, w_dist: str, b_dist: str, seed: int) -> Tensors:
    rng = np.random.default_rng(seed)
    xs = tuple(int(v) for v in x_shape)
    ws = tuple(int(v) for v in w_shape)
    x = _draw(rng, x_dist, int(np.prod(xs))).reshape(xs).astype(np.float32)
    w = _draw(rng, w_dist, int(np.prod(ws))).reshape(ws).astype(np.float32)
    b = _draw(rng, b_dist, int(c_out)).astype(np.float32) if has_bias else None
    if dtype == "f32":
        return Tensors("f32", x, w, b, x, w, b)
    if dtype == "bf16":
        xb, wb = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
        bb = f32_to_bf16_bits(b) if b is not None else None
        return Tensors("bf16", bf16_bits_to_f32(xb).reshape(xs), bf16_bits_to_f32(wb).reshape(ws),
                       bf16_bits_to_f32(bb) if bb is not None else None,
                       xb.reshape(xs), wb.reshape(ws), bb)
    if dtype == "f16":
        # IEEE half, round to nearest even (numpy's conversion)
        xh, wh = x.astype(np.float16), w.astype(np.float16)
        bh = b.astype(np.float16) if b is not None else None
        return Tensors("f16", xh.astype(np.float32), wh.astype(np.float32),
                       bh.astype(np.float32) if bh is not None else None,
                       xh.view(np.uint16), wh.view(np.uint16),
                       bh.view(np.uint16) if bh is not None else None)
    raise ValueError(f"unknown dtype {dtype!r}")


def workload_tensors(wl: Workload, seed: Optional[int] = None) -> Tensors:
    return make_tensors(wl.x_shape, wl.w_shape, wl.c_out, wl.has_bias, wl.dtype,
                        wl.x_dist, wl.w_dist, wl.b_dist, wl.seed if seed is None else seed)
