"""CPU tests of the C ABI: the library loads and exports what include/convt.h
declares, the planner validates and sizes problems (host only, no device call),
the stride-phase tables have the properties the phase split relies on, and the
entry points refuse bad arguments before touching the device."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import convt_forward_amd as C
import oracle
import workloads
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convt.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(convt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = C.lib()
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in convt.h but not exported"


def test_status_and_route_names():
    L = C.lib()
    assert L.convt_status_string(0) == b"ok"
    assert L.convt_status_string(1) == b"invalid argument"
    assert L.convt_status_string(2) == b"unsupported request"
    assert L.convt_status_string(3) == b"device error"
    for name, code in C.ROUTES.items():
        assert L.convt_route_name(code).decode() == name
    assert L.convt_version() >= 200


def plan(**kw):
    base = dict(x_shape=(1, 1, 3), w_shape=(1, 2, 2), stride=1, padding=0, dilation=1,
                output_padding=0, groups=1, has_bias=False, dtype="f32", route="auto")
    base.update(kw)
    return C.Plan.create(**base)


def status_of(**kw):
    try:
        plan(**kw)
    except C.ConvtError as e:
        return e.status
    return 0


def test_page_example_shape():
    # huggingface ai.onnx.ConvTranspose usage example: x [1,1,3], w [1,2,2], defaults
    assert plan().out_shape == (1, 2, 4)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_workload_plans(name):
    wl = workloads.get(name)
    pl = plan(x_shape=wl.x_shape, w_shape=wl.w_shape, stride=wl.stride, padding=wl.padding,
              dilation=wl.dilation, output_padding=wl.output_padding, groups=wl.groups,
              has_bias=wl.has_bias, dtype=wl.dtype)
    assert pl.out_shape == oracle.out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.padding,
                                            wl.dilation, wl.output_padding, wl.groups)
    expect_route = {"c1_2d_f32_small": "direct", "c2_1d_f32_upsampler": "phase_gemm",
                    "c3_2d_bf16_generator": "phase_gemm_allphase", "c4a_2d_bf16_grouped": "grouped",
                    "c4b_2d_bf16_dilated": "phase_gemm", "c5_3d_bf16_video": "phase_gemm_allphase"}[name]
    assert pl.route == expect_route
    b, cin = wl.x_shape[:2]
    assert pl.useful_flops == 2 * b * cin * wl.w_shape[1] * int(np.prod(wl.w_shape[2:])) * int(
        np.prod(wl.x_shape[2:]))
    assert pl.n_phases == int(np.prod(wl.stride))


def test_plan_shapes_match_oracle_on_random_grid():
    rng = np.random.default_rng(5)
    for prm in oracle_pins.random_grid(rng, 300):
        xs = (prm["B"], prm["Ci"]) + tuple(prm["I"])
        ws = (prm["Ci"], prm["Cog"]) + tuple(prm["k"])
        pad = tuple(zip(prm["p"], prm["ph"]))
        pl = plan(x_shape=xs, w_shape=ws, stride=prm["s"], padding=pad, dilation=prm["d"],
                  output_padding=prm["op"], groups=prm["groups"])
        assert pl.out_shape == oracle.out_shape(xs, ws, prm["s"], pad, prm["d"], prm["op"],
                                                prm["groups"])


REJECT = [
    # SKaiNET convTranspose2d page, validation rules
    dict(output_padding=1),                                 # op must be < max(stride, dilation) = 1
    dict(stride=2, output_padding=2),                       # op == stride
    dict(x_shape=(1, 3, 4), w_shape=(3, 1, 2), groups=2),   # groups must divide C_in
    dict(x_shape=(1, 2, 4), w_shape=(3, 1, 2)),             # C_in of x and W differ
    dict(stride=0),
    dict(dilation=0),
    dict(padding=-1),
    dict(output_padding=-1),
    dict(groups=0),
    dict(x_shape=(1, 1, 1), w_shape=(1, 1, 1), padding=1),  # output size (1-1)*1 - 2 + 0 + 1 < 1
    dict(padding=((0, -1),)),                               # negative high padding
    dict(x_shape=(1, 1, 2), w_shape=(1, 1, 2), padding=((0, 3),)),  # 1 - 3 + 1 + 1 < 1
    dict(w_shape=(1, 2, 0)),                                # empty kernel
    dict(x_shape=(-1, 1, 3)),
]


@pytest.mark.parametrize("kw", REJECT)
def test_plan_rejects_invalid(kw):
    assert status_of(**kw) == 1


# valid problems whose per-axis index terms exceed 32 bits: refused as
# unsupported rather than indexed with wrapped arithmetic
TOO_WIDE = [
    # output size (1048676-1) - 2*2^39 + 2^20*(2^20-1) + 1 = 100
    dict(x_shape=(1, 1, 1048676), w_shape=(1, 1, 1048576), padding=2 ** 39, dilation=2 ** 20),
    # low padding 2^31, high padding 0
    dict(x_shape=(1, 1, 2 ** 12), w_shape=(1, 1, 2 ** 12), padding=((2 ** 31, 0),), dilation=2 ** 20),
    # (2^31 - 1) * 2 + 1 output positions
    dict(x_shape=(1, 1, 2 ** 31), w_shape=(1, 1, 1), stride=2),
]


@pytest.mark.parametrize("kw", TOO_WIDE)
def test_plan_refuses_int32_overflowing_axes(kw):
    assert status_of(**kw) == 2


@pytest.mark.parametrize("dt", ["i8", "i32", "i64"])
def test_plan_refuses_other_dtypes_loudly(dt):
    assert status_of(dtype=dt) == 2


def test_plan_rejects_malformed_struct():
    p = C.make_problem((1, 1, 3), (1, 2, 2))
    for field, val in [("ndim", 0), ("ndim", 4), ("has_bias", 2), ("route", 99), ("dtype", 42)]:
        q = C.make_problem((1, 1, 3), (1, 2, 2))
        setattr(q, field, val)
        h = ctypes.c_void_p()
        st = C.lib().convt_plan(ctypes.byref(q), ctypes.byref(h), None)
        assert st == 1, (field, val)
        assert not h.value
    h = ctypes.c_void_p(1234)
    assert C.lib().convt_plan(None, ctypes.byref(h), None) == 1
    assert not h.value
    assert C.lib().convt_plan(ctypes.byref(p), None, None) == 1


def test_edge_routes():
    assert plan(x_shape=(0, 1, 3)).route == "none"                       # empty batch
    assert plan(x_shape=(2, 0, 3), w_shape=(0, 2, 2)).route == "fill"    # no input channels
    pl = plan(x_shape=(2, 3, 0), w_shape=(3, 2, 3), has_bias=True)       # empty input axis
    assert pl.out_shape == (2, 2, 2) and pl.route == "fill"
    assert plan(x_shape=(1, 2, 4), w_shape=(2, 3, 2), stride=17).route in ("naive", "direct")
    # stride 17 is beyond the phase tables: only the naive route serves it
    assert plan(x_shape=(1, 64, 4), w_shape=(64, 64, 2), stride=17).route == "naive"


def test_forced_routes():
    # grouped needs bfloat16 and groups of 8k channels
    assert status_of(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, groups=2,
                     route="grouped") == 2
    assert plan(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, groups=2, dtype="bf16",
                route="grouped").route == "grouped"
    assert plan(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, route="naive").route == "naive"
    assert status_of(x_shape=(0, 1, 3), route="naive") == 2   # nothing to compute
    assert status_of(x_shape=(1, 64, 4), w_shape=(64, 64, 2), stride=17, route="phase_gemm") == 2
    # the packed phase GEMM serves two-byte types only, and only forward
    assert status_of(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2,
                     route="phase_gemm_packed") == 2
    assert plan(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, dtype="bf16",
                route="phase_gemm_packed").route == "phase_gemm_packed"
    assert status_of(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, dtype="bf16",
                     route_bwd="phase_gemm_packed") == 2
    # a two-byte problem the in-place kernel does not suit (odd input rows)
    # is planned on the packed variant when PHASE_GEMM is asked for
    assert plan(x_shape=(2, 72, 9, 13), w_shape=(72, 136, 4, 4), stride=2, padding=1, dtype="bf16",
                route="phase_gemm").route == "phase_gemm_packed"


def test_workspace_sizes():
    wl = workloads.get("c3")
    # the all-phase kernel (the automatic choice here) reads W as stored
    ap = plan(x_shape=wl.x_shape, w_shape=wl.w_shape, stride=wl.stride, padding=wl.padding,
              dtype="bf16", has_bias=True)
    assert ap.route == "phase_gemm_allphase" and ap.workspace_bytes == 0
    pl = plan(x_shape=wl.x_shape, w_shape=wl.w_shape, stride=wl.stride, padding=wl.padding,
              dtype="bf16", has_bias=True, route="phase_gemm")
    # reordered weights (no padding needed at these sizes) and the per-tap
    # halo shift table (16 taps of 4 bytes); the bfloat16 GEMM reads x in
    # place
    assert pl.route == "phase_gemm"
    wr_bytes = 512 * 256 * 16 * 2
    assert pl.workspace_bytes == wr_bytes + 16 * 4
    # the packed variant adds the channel-chunked copy of x it reads
    pk = plan(x_shape=wl.x_shape, w_shape=wl.w_shape, stride=wl.stride, padding=wl.padding,
              dtype="bf16", has_bias=True, route="phase_gemm_packed")
    assert pk.route == "phase_gemm_packed"
    # (after the table's 256-byte aligned slot)
    assert pk.workspace_bytes == wr_bytes + 256 + 64 * 512 * 16 * 16 * 2
    pl = plan(x_shape=(1, 3, 5), w_shape=(3, 5, 3), stride=2, route="phase_gemm")
    # channels padded to the f32 tile: 16 input (two 8-channel chunks per
    # stage), 64 output, 3 taps (phases of 2 and 1 taps, one tap per stage);
    # then the tap table, 4 bytes per tap
    assert pl.workspace_bytes == 1 * 3 * 64 * 16 * 4 + 3 * 4
    assert plan(x_shape=(1, 3, 5), w_shape=(3, 5, 3), route="naive").workspace_bytes == 0


def test_phase_table_properties():
    """For every residue r: taps kk with (r + p - kk*d) divisible by s, each
    with offset (r + p - kk*d)/s, ascending; the residues partition the taps
    and their q counts partition the outputs."""
    rng = np.random.default_rng(6)
    for prm in oracle_pins.random_grid(rng, 200):
        xs = (prm["B"], prm["Ci"]) + tuple(prm["I"])
        ws = (prm["Ci"], prm["Cog"]) + tuple(prm["k"])
        pl = plan(x_shape=xs, w_shape=ws, stride=prm["s"], padding=tuple(zip(prm["p"], prm["ph"])),
                  dilation=prm["d"],
                  output_padding=prm["op"], groups=prm["groups"])
        for a in range(prm["nd"]):
            s, p, d, k = prm["s"][a], prm["p"][a], prm["d"][a], prm["k"][a]
            O = pl.out_shape[2 + a]
            seen, qsum = [], 0
            for r in range(s):
                q, taps, offs = pl.axis_phase(a, r)
                qsum += q
                assert q == len(range(r, O, s))
                assert offs == sorted(offs)
                for kk, off in zip(taps, offs):
                    assert 0 <= kk < k
                    assert r + p - kk * d == off * s
                assert sorted(taps) == [kk for kk in range(k) if (r + p - kk * d) % s == 0]
                seen += taps
            assert sorted(seen) == list(range(k))
            assert qsum == O


def test_allphase_route_rules():
    """The all-phase route takes two-byte problems with stride 2 and
    dilation 1 on the two innermost axes, 4 or 8 taps per phase, an even x
    row and an output row length that is a multiple of 8; it is refused
    otherwise."""
    ok = dict(x_shape=(1, 16, 6, 16), w_shape=(16, 96, 4, 4), stride=2, padding=1, dtype="bf16")
    assert plan(**ok, route="phase_gemm_allphase").route == "phase_gemm_allphase"
    assert plan(**ok).route == "phase_gemm_allphase"
    assert plan(**dict(ok, dtype="f16"), route="phase_gemm_allphase").workspace_bytes == 0
    for bad in [dict(dtype="f32"), dict(stride=(2, 1)), dict(dilation=2), dict(x_shape=(1, 16, 6, 15)),
                dict(padding=(1, 0)),                                    # output rows of 34
                dict(w_shape=(16, 96, 3, 3)), dict(w_shape=(16, 96, 2, 2)),
                dict(x_shape=(1, 16, 16), w_shape=(16, 96, 4), stride=2, padding=1),  # 1-D
                dict(filter_layout="k_ci_co")]:
        assert status_of(**dict(ok, **bad), route="phase_gemm_allphase") == 2, bad
    # 64 or fewer output channels per group: the automatic choice is another kernel
    assert plan(**dict(ok, w_shape=(16, 64, 4, 4))).route != "phase_gemm_allphase"
    # host-side refusals: x must be 4-byte and W 16-byte aligned
    L = C.lib()
    h = plan(**ok, has_bias=False).handle
    fake = 4096
    assert L.convt_forward(h, fake + 2, fake, None, fake, None, None) == 1
    assert L.convt_forward(h, fake, fake + 8, None, fake, None, None) == 1
    assert L.convt_forward_prepared(h, fake, fake + 8, None, fake, None, None) == 1
    assert L.convt_forward_prepared(h, fake, None, None, fake, None, None) == 1


def test_forward_refuses_bad_arguments_before_launch():
    """Each call below fails a host-side check, so nothing reaches the device."""
    L = C.lib()
    pl = plan(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, has_bias=True, route="phase_gemm")
    h = pl.handle
    fake = 4096  # never dereferenced: every call fails an argument check first
    assert L.convt_forward(None, fake, fake, fake, fake, fake, None) == 1
    assert L.convt_forward(h, fake, fake, None, fake, fake, None) == 1          # bias required
    assert L.convt_forward(h, fake, fake, fake, None, fake, None) == 1          # y required
    assert L.convt_forward(h, None, fake, fake, fake, fake, None) == 1          # x required
    assert L.convt_forward(h, fake, fake, fake, fake, None, None) == 1          # workspace required
    assert L.convt_forward(h, fake, fake, fake, fake, fake + 8, None) == 1      # misaligned workspace
    assert L.convt_prepare_weights(h, fake, None, None) == 1
    assert L.convt_prepare_weights(None, fake, fake, None) == 1
    assert L.convt_forward_prepared(h, fake, fake, None, fake, fake, None) == 1
    assert L.convt_forward_prepared(None, fake, fake, fake, fake, fake, None) == 1
    pl2 = plan(x_shape=(1, 16, 8), w_shape=(16, 8, 4), stride=2, has_bias=False, route="naive")
    assert L.convt_forward(pl2.handle, fake, fake, fake, fake, None, None) == 1  # unexpected bias
    # an empty output needs no pointers at all
    pl3 = plan(x_shape=(0, 16, 8), w_shape=(16, 8, 4), stride=2)
    assert L.convt_forward(pl3.handle, None, None, None, None, None, None) == 0
    L.convt_destroy(None)


def test_axis_phase_arguments():
    pl = plan(x_shape=(1, 1, 5), w_shape=(1, 1, 4), stride=2, padding=1)
    q = ctypes.c_int64()
    n = ctypes.c_int64()
    assert C.lib().convt_plan_axis_phase(pl.handle, 1, 0, ctypes.byref(q), ctypes.byref(n),
                                         None, None, 0) == 1   # axis out of range
    assert C.lib().convt_plan_axis_phase(pl.handle, 0, 2, ctypes.byref(q), ctypes.byref(n),
                                         None, None, 0) == 1   # residue out of range
    assert C.lib().convt_plan_axis_phase(pl.handle, 0, 1, ctypes.byref(q), ctypes.byref(n),
                                         None, None, 0) == 0
    assert (q.value, n.value) == (5, 2)


def test_problem_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of convt_problem has the header's size and offsets
    (compiled from include/convt.h with the host C compiler)."""
    fields = [f[0] for f in C.Problem._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"convt.h\"\nint main(void){\n"
                   "printf(\"%zu\\n\", sizeof(convt_problem));\n"
                   + "".join("printf(\"%%zu\\n\", offsetof(convt_problem, %s));\n" % f for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(t) for t in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(C.Problem)
    assert out[1:] == [getattr(C.Problem, f).offset for f in fields]


def test_padding_hi_fields_validated():
    L = C.lib()
    for has_hi, rb, hi, want in [(2, 0, 0, 1), (0, 99, 0, 1), (1, 0, -1, 1), (1, 0, 1, 0), (1, 0, 3, 0),
                                  (0, 0, -5, 0)]:
        p = C.make_problem((1, 1, 4), (1, 1, 3), stride=2, padding=1)
        p.has_padding_hi, p.route_bwd, p.padding_hi[0] = has_hi, rb, hi
        h = ctypes.c_void_p()
        info = C.PlanInfo()
        st = L.convt_plan(ctypes.byref(p), ctypes.byref(h), ctypes.byref(info))
        assert st == want, (has_hi, rb, hi, st)
        if st == 0:
            # (4-1)*2 - (1 + p_hi) + (3-1) + 1, p_hi read only when has_padding_hi is 1
            assert info.out_shape[2] == 8 - (hi if has_hi else 1)
            L.convt_destroy(h)


def test_backward_data_refuses_bad_arguments_before_launch():
    """Host-side checks of convt_backward_data: nothing reaches the device."""
    L = C.lib()
    pl = plan(x_shape=(1, 32, 8), w_shape=(32, 16, 4), stride=2)
    assert pl.route_bwd == "phase_gemm" and pl.bwd_workspace_bytes > 0
    h = pl.handle
    fake = 4096  # never dereferenced
    assert L.convt_backward_data(None, fake, fake, fake, fake, None) == 1
    assert L.convt_backward_data(h, fake, fake, None, fake, None) == 1        # dx required
    assert L.convt_backward_data(h, None, fake, fake, fake, None) == 1        # dy required
    assert L.convt_backward_data(h, fake, None, fake, fake, None) == 1        # w required
    assert L.convt_backward_data(h, fake, fake, fake, None, None) == 1        # workspace required
    assert L.convt_backward_data(h, fake, fake, fake, fake + 8, None) == 1    # misaligned


def test_allphase_backward_route_rules():
    """The backward all-phase kernel takes two-byte problems with stride 2
    and dilation 1 on the two innermost axes, 16 taps over them (4x4, 2x8,
    8x2), an even dy row and a dx row length that is a multiple of 8, W in
    the C_in x C_out x taps layout; no workspace. The automatic choice takes
    it for more than 64 dx channels per group."""
    ok = dict(x_shape=(1, 96, 6, 16), w_shape=(96, 24, 4, 4), stride=2, padding=1, dtype="bf16")
    pl = plan(**ok)
    assert pl.route_bwd == "phase_gemm_allphase" and pl.bwd_workspace_bytes == 0
    for good in [dict(), dict(dtype="f16"), dict(w_shape=(96, 24, 2, 8)), dict(w_shape=(96, 24, 8, 2)),
                 dict(padding=(0, 2)), dict(padding=((1, 3), (0, 2))), dict(groups=2, w_shape=(96, 8, 4, 4)),
                 dict(x_shape=(1, 96, 3, 6, 16), w_shape=(96, 24, 3, 4, 4), stride=(1, 2, 2), padding=1),
                 dict(x_shape=(1, 96, 3, 6, 16), w_shape=(96, 24, 4, 4, 4), stride=2, padding=1)]:
        assert plan(**dict(ok, **good), route_bwd="phase_gemm_allphase").route_bwd == "phase_gemm_allphase"
    for bad in [dict(dtype="f32"), dict(stride=(2, 1)), dict(dilation=2), dict(x_shape=(1, 96, 6, 12)),
                dict(output_padding=(0, 1)),                              # dy rows of 33
                dict(w_shape=(96, 24, 3, 3)), dict(w_shape=(96, 24, 4, 8)), dict(w_shape=(96, 24, 2, 2)),
                dict(x_shape=(1, 96, 16), w_shape=(96, 24, 4), stride=2, padding=1),  # 1-D
                dict(filter_layout="k_ci_co")]:
        assert status_of(**dict(ok, **bad), route_bwd="phase_gemm_allphase") == 2, bad
    # 64 or fewer dx channels per group: the automatic choice is another kernel
    assert plan(**dict(ok, x_shape=(1, 64, 6, 16), w_shape=(64, 24, 4, 4))).route_bwd == "phase_gemm"
    # the forward's packed route has no backward counterpart
    assert status_of(**ok, route_bwd="phase_gemm_packed") == 2
    # host-side refusals: dy must be 4-byte, W and dx 16-byte aligned
    L = C.lib()
    h = pl.handle
    fake = 4096  # never dereferenced
    assert L.convt_backward_data(h, fake + 2, fake, fake, None, None) == 1
    assert L.convt_backward_data(h, fake, fake + 8, fake, None, None) == 1
    assert L.convt_backward_data(h, fake, fake, fake + 8, None, None) == 1


def test_grouped_backward_route_rules():
    """route_bwd GROUPED: two-byte 2-D problems with output channels per group
    a multiple of 8 (at most 16 (tap, 8-channel slice) slots), at most 16
    input channels per group and dy rows of whole 16-byte chunks; AUTO takes
    it there (the grouped workload), forced elsewhere it is refused."""
    wl = workloads.get("c4a")
    assert plan(x_shape=wl.x_shape, w_shape=wl.w_shape, stride=wl.stride, padding=wl.padding,
                groups=wl.groups, dtype="bf16").route_bwd == "grouped"
    ok = dict(x_shape=(1, 16, 9, 16), w_shape=(16, 8, 4, 4), stride=2, padding=1, groups=2, dtype="bf16")
    assert plan(**ok).route_bwd == "grouped"
    assert plan(**dict(ok, dtype="f16")).route_bwd == "grouped"
    for bad in (dict(dtype="f32"),                                        # element type
                dict(w_shape=(16, 4, 4, 4)),                              # Cog not a multiple of 8
                dict(x_shape=(1, 34, 9, 16), w_shape=(34, 8, 4, 4)),      # 17 input channels per group
                dict(w_shape=(16, 24, 4, 4)),                             # 3 slices x 16 taps > 16 slots
                dict(x_shape=(1, 16, 9, 15)),                             # dy rows of 30 values
                dict(x_shape=(1, 16, 3, 9, 16), w_shape=(16, 8, 2, 4, 4), stride=(1, 2, 2),
                     padding=(0, 1, 1))):                                 # 3-D
        assert status_of(**dict(ok, **bad), route_bwd="grouped") == 2, bad
        assert plan(**dict(ok, **bad)).route_bwd != "grouped", bad


def test_backward_routes():
    """Routes of the backward pass: forced routes that cannot serve are
    refused; the naive route serves any problem; few channels per group take
    the direct kernel (any stride), many the GEMM."""
    assert plan(x_shape=(0, 2, 5), w_shape=(2, 3, 3)).route_bwd == "none"
    assert plan(x_shape=(1, 2, 5), w_shape=(2, 0, 3)).route_bwd == "fill"
    assert plan(x_shape=(1, 2, 5), w_shape=(2, 3, 3)).route_bwd == "direct"
    assert plan(x_shape=(1, 2, 5), w_shape=(2, 3, 3), stride=19).route_bwd == "direct"
    assert plan(x_shape=(1, 64, 5), w_shape=(64, 64, 3), stride=19).route_bwd == "naive"
    assert plan(x_shape=(1, 64, 5), w_shape=(64, 64, 3), stride=2).route_bwd == "phase_gemm"
    assert plan(x_shape=(1, 64, 5), w_shape=(64, 32, 3), route_bwd="direct").route_bwd == "direct"
    # the direct kernel's weights (64 x 64 x 3 float32 = 48 KiB, plus the tap
    # table) exceed its LDS
    assert status_of(x_shape=(1, 64, 5), w_shape=(64, 64, 3), route_bwd="direct") == 2
    assert plan(x_shape=(1, 2, 5), w_shape=(2, 3, 3), route_bwd="naive").route_bwd == "naive"
    assert status_of(x_shape=(1, 2, 5), w_shape=(2, 3, 3), stride=19, route_bwd="phase_gemm") == 2
    assert status_of(x_shape=(1, 2, 5), w_shape=(2, 3, 3), route_bwd="fill") == 2
    assert status_of(x_shape=(1, 2, 5), w_shape=(2, 3, 3), route_bwd="grouped") == 2


def test_filter_layout_shapes_and_validation():
    """W's shape in each filter layout (include/convt.h) and back; bad codes
    are refused."""
    ws = (6, 5, 3, 4)  # C_in 6, C_out/groups 5, k 3x4, groups 2
    assert C.layout_w_shape(ws, 2, "ci_co_k") == ws
    assert C.layout_w_shape(ws, 2, "k_ci_co") == (3, 4, 6, 5)
    assert C.layout_w_shape(ws, 2, "k_co_ci") == (3, 4, 10, 3)
    for lay in C.FILTER_LAYOUTS:
        assert C.canonical_w_shape(C.layout_w_shape(ws, 2, lay), 2, lay) == ws
    L = C.lib()
    for fl, tf in [(3, 0), (-1, 0), (0, 2)]:
        p = C.make_problem((1, 6, 5, 5), ws, groups=2)
        p.filter_layout, p.taps_flipped = fl, tf
        h = ctypes.c_void_p()
        assert L.convt_plan(ctypes.byref(p), ctypes.byref(h), None) == 1
    pl = plan(x_shape=(1, 6, 5, 5), w_shape=ws, groups=2, filter_layout="k_co_ci", taps_flipped=True)
    assert pl.w_layout_shape == (3, 4, 10, 3)


def test_activation_and_reserved_fields_validated():
    L = C.lib()
    for act, res, want in [(6, 0, 1), (-1, 0, 1), (0, 1, 1), (5, 0, 0), (0, 0, 0)]:
        p = C.make_problem((1, 2, 5), (2, 3, 3), stride=2, dtype="f16")
        p.activation, p.reserved1 = act, res
        h = ctypes.c_void_p()
        st = L.convt_plan(ctypes.byref(p), ctypes.byref(h), None)
        assert st == want, (act, res, st)
        if st == 0:
            L.convt_destroy(h)


def test_scratch_entry_point_host_checks():
    """convt_forward_scratch: the limit, and refusals made before any device
    call (a plan whose workspace exceeds the library's array)."""
    L = C.lib()
    assert L.convt_scratch_max_bytes() == 32 * 1024 * 1024
    fake = 4096  # never dereferenced: every call below fails a host-side check
    assert L.convt_forward_scratch(None, fake, fake, fake, fake, None) == 1
    big = plan(x_shape=(1, 2048, 4, 4), w_shape=(2048, 1024, 4, 4), stride=2, padding=1,
               dtype="bf16", has_bias=True, route="phase_gemm")
    assert big.workspace_bytes > L.convt_scratch_max_bytes()
    assert L.convt_forward_scratch(big.handle, fake, fake, fake, fake, None) == 2
    # convt_plan_query reports what convt_plan did
    info = C.PlanInfo()
    assert L.convt_plan_query(big.handle, ctypes.byref(info)) == 0
    assert info.workspace_bytes == big.workspace_bytes and info.route == big.info.route
    assert L.convt_plan_query(big.handle, None) == 1
