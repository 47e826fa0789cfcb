"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``check_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages and the mathematics fix. They are
run as ordinary CPU tests against the oracle as built, and against deliberately
broken builds of its C source (every such mutant must fail at least one check).

What pins what:
  * hand-computed golden cases (tests/golden/*.json): the 'k2/s1 full scatter'
    and 'k2/s2 non-overlapping stamp' cases named in the SKaiNET
    convTranspose2d pull request (Tests), plus stride-2/pad-1/output_padding-1,
    dilation-2, groups-2 and multi-channel points of the parameter grid it
    names, all worked by hand;
  * output sizes against the closed form evaluated by hand (same page's
    Summary; AWS Neuron conv3d_transpose page, Dimensions);
  * stride 1 / pad 0 / dilation 1 single-channel results equal scipy's full
    convolution (a textbook identity);
  * kernel == stride, pad 0: each input sample stamps a disjoint scaled copy
    of the kernel, i.e. numpy.kron;
  * 1x1 kernels: a per-pixel matrix product, zero-inserted when stride > 1;
  * the lowering the pages describe (SKaiNET Summary, StableHLO lowering;
    AWS Neuron page, Background): a stride-1 forward convolution of the input
    with stride-1 zeros inserted between samples, taps flipped, padding
    dilation*(k-1) - padding on the low side and that plus output_padding on
    the high side (negative = crop), groups handled one at a time;
  * the adjoint identity <convT(x, W), y> = <x, conv(y, W)>, with conv the
    strided forward convolution written as a gather;
  * groups == concatenation of ungrouped per-group problems; exact bias
    offset and linearity on integer data; conservation of the total sum when
    nothing is cropped;
  * brute force: pure-Python enumeration of every (input position, tap) pair
    per output on tiny problems;
  * the per-output magnitude sum equals the transposed convolution of |x|, |W|;
  * the single-point evaluation agrees with the full pass;
  * results do not depend on the thread count; ill-formed problems are refused.
"""
from __future__ import annotations

import glob
import itertools
import json
import os

import numpy as np
import scipy.signal

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Independent helpers (none of them calls the oracle)
# ---------------------------------------------------------------------------

def _pad_or_crop(a: np.ndarray, axis: int, lo: int, hi: int) -> np.ndarray:
    """Zero-pad (positive) or crop (negative) ``lo`` at the start and ``hi`` at
    the end of ``axis``."""
    if lo < 0:
        a = np.take(a, np.arange(-lo, a.shape[axis]), axis=axis)
    if hi < 0:
        a = np.take(a, np.arange(0, a.shape[axis] + hi), axis=axis)
    widths = [(0, 0)] * a.ndim
    widths[axis] = (max(lo, 0), max(hi, 0))
    return np.pad(a, widths)


def lowered_reference(x, w, bias, s, p, d, op, groups, ph=None):
    """Transposed convolution via the lowering on the pages: dilate the input by
    the stride (stride-1 zeros between samples), pad low d*(k-1)-p and high
    d*(k-1)-p_hi+op (p_hi = p when the padding is symmetric), flip the taps,
    then a stride-1 dilated forward correlation, one group at a time."""
    ph = p if ph is None else ph
    nd = x.ndim - 2
    B, Ci = x.shape[:2]
    Cig, Cog = Ci // groups, w.shape[1]
    k = w.shape[2:]
    dshape = (B, Ci) + tuple((I - 1) * sa + 1 for I, sa in zip(x.shape[2:], s))
    xd = np.zeros(dshape)
    xd[(slice(None), slice(None)) + tuple(slice(None, None, sa) for sa in s)] = x
    for a in range(nd):
        lo = d[a] * (k[a] - 1) - p[a]
        hi = d[a] * (k[a] - 1) - ph[a] + op[a]
        xd = _pad_or_crop(xd, 2 + a, lo, hi)
    wf = w[(slice(None), slice(None)) + (slice(None, None, -1),) * nd]
    out_sp = tuple(xd.shape[2 + a] - d[a] * (k[a] - 1) for a in range(nd))
    y = np.zeros((B, Cog * groups) + out_sp)
    for g in range(groups):
        xg = xd[:, g * Cig:(g + 1) * Cig]
        wg = wf[g * Cig:(g + 1) * Cig]
        for kk in itertools.product(*[range(t) for t in k]):
            sl = tuple(slice(kk[a] * d[a], kk[a] * d[a] + out_sp[a]) for a in range(nd))
            win = xg[(slice(None), slice(None)) + sl]
            tap = wg[(slice(None), slice(None)) + kk]
            y[:, g * Cog:(g + 1) * Cog] += np.tensordot(win, tap, axes=([1], [0])).transpose(
                (0, nd + 1) + tuple(range(1, nd + 1)))
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64).reshape((1, -1) + (1,) * nd)
    return y


def forward_conv_gather(yv, w, s, p, d, in_sp, groups):
    """Strided forward convolution written as a gather (the adjoint of the
    transposed convolution): out[b, ci, i] = sum over oc in the group of ci and
    taps kk of y[b, oc, i*s - p + kk*d] * W[ci, oc - g*Cog, kk], with y taken as
    zero outside its extent."""
    nd = yv.ndim - 2
    B, Co = yv.shape[:2]
    Ci, Cog = w.shape[0], w.shape[1]
    Cig = Ci // groups
    k = w.shape[2:]
    out = np.zeros((B, Ci) + tuple(in_sp))
    for g in range(groups):
        yg = yv[:, g * Cog:(g + 1) * Cog]
        wg = w[g * Cig:(g + 1) * Cig]
        for kk in itertools.product(*[range(t) for t in k]):
            idx, mask = [], None
            for a in range(nd):
                pos = np.arange(in_sp[a]) * s[a] - p[a] + kk[a] * d[a]
                ok = (pos >= 0) & (pos < yv.shape[2 + a])
                idx.append(np.clip(pos, 0, yv.shape[2 + a] - 1))
                m = ok.reshape([-1 if j == a else 1 for j in range(nd)])
                mask = m if mask is None else mask & m
            sel = yg[(slice(None), slice(None)) + np.ix_(*idx)] * mask
            tap = wg[(slice(None), slice(None)) + kk]  # [Cig, Cog]
            out[:, g * Cig:(g + 1) * Cig] += np.tensordot(sel, tap, axes=([1], [1])).transpose(
                (0, nd + 1) + tuple(range(1, nd + 1)))
    return out


def brute_force(x, w, bias, s, p, d, op, groups, ph=None):
    """Every output by enumerating all (input position, tap) pairs in Python;
    the low padding p shifts the outputs, the high padding p_hi only shortens
    the axis."""
    ph = p if ph is None else ph
    nd = x.ndim - 2
    B, Ci = x.shape[:2]
    Cig, Cog = Ci // groups, w.shape[1]
    k = w.shape[2:]
    I = x.shape[2:]
    O = tuple((I[a] - 1) * s[a] - p[a] - ph[a] + d[a] * (k[a] - 1) + op[a] + 1
              for a in range(nd))
    y = np.zeros((B, Cog * groups) + O)
    for b in range(B):
        for oc in range(Cog * groups):
            g = oc // Cog
            for o in itertools.product(*[range(t) for t in O]):
                acc = float(bias[oc]) if bias is not None else 0.0
                for ci in range(g * Cig, (g + 1) * Cig):
                    for i in itertools.product(*[range(t) for t in I]):
                        for kk in itertools.product(*[range(t) for t in k]):
                            if all(i[a] * s[a] - p[a] + kk[a] * d[a] == o[a] for a in range(nd)):
                                acc += float(x[(b, ci) + i]) * float(w[(ci, oc - g * Cog) + kk])
                y[(b, oc) + o] = acc
    return y


def _rand_problem(rng, nd, B, Ci, Cog, groups, I, k, s, p, d, op, bias=True, ints=False,
                  ph=None):
    Ci_t = Ci
    if ints:
        x = rng.integers(-4, 5, size=(B, Ci_t) + tuple(I)).astype(np.float64)
        w = rng.integers(-4, 5, size=(Ci_t, Cog) + tuple(k)).astype(np.float64)
        b = rng.integers(-4, 5, size=(Cog * groups,)).astype(np.float64) if bias else None
    else:
        x = rng.standard_normal((B, Ci_t) + tuple(I))
        w = rng.standard_normal((Ci_t, Cog) + tuple(k))
        b = rng.standard_normal(Cog * groups) if bias else None
    pad = tuple(p) if ph is None or list(ph) == list(p) else tuple(zip(p, ph))
    return x, w, b, dict(stride=tuple(s), padding=pad, dilation=tuple(d),
                         output_padding=tuple(op), groups=groups)


def _close(a, b, rtol=1e-12, atol=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b) / (np.abs(b) + 1.0)) if a.size else 0.0
    assert err <= max(rtol, atol), f"max relative error {err}"


def random_grid(rng, n, nds=(1, 2, 3), asym=True):
    """Seeded random valid parameter sets (output_padding < max(stride,
    dilation)), including pads beyond d*(k-1) and phases with no taps. With
    asym, about half the sets get a high padding ``ph`` that differs from the
    low one on some axis; otherwise ``ph`` equals ``p``."""
    out = []
    while len(out) < n:
        nd = int(rng.choice(nds))
        groups = int(rng.choice([1, 1, 2, 3]))
        Cig = int(rng.integers(1, 4))
        Cog = int(rng.integers(1, 4))
        B = int(rng.integers(1, 3))
        I = [int(rng.integers(1, 6 if nd < 3 else 4)) for _ in range(nd)]
        k = [int(rng.integers(1, 5 if nd < 3 else 4)) for _ in range(nd)]
        s = [int(rng.integers(1, 5)) for _ in range(nd)]
        d = [int(rng.integers(1, 4)) for _ in range(nd)]
        p = [int(rng.integers(0, d[a] * (k[a] - 1) + 2)) for a in range(nd)]
        op = [int(rng.integers(0, max(s[a], d[a]))) for a in range(nd)]
        ph = list(p)
        if asym and rng.integers(0, 2):
            ph = [int(rng.integers(0, d[a] * (k[a] - 1) + 2)) for a in range(nd)]
        O = [(I[a] - 1) * s[a] - p[a] - ph[a] + d[a] * (k[a] - 1) + op[a] + 1 for a in range(nd)]
        if min(O) < 1:
            continue
        out.append(dict(nd=nd, B=B, Ci=Cig * groups, Cog=Cog, groups=groups, I=I, k=k, s=s, p=p,
                        ph=ph, d=d, op=op))
    return out


# ---------------------------------------------------------------------------
# Checks
# ---------------------------------------------------------------------------

def check_golden_cases(orc):
    files = sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json")))
    n = 0
    for f in files:
        case = json.load(open(f))
        if "y" not in case:
            continue
        x = np.array(case["x"], dtype=np.float64).reshape(case["x_shape"])
        w = np.array(case["w"], dtype=np.float64).reshape(case["w_shape"])
        b = np.array(case["bias"], dtype=np.float64) if case["bias"] is not None else None
        y, _ = orc.forward(x, w, b, case["stride"], case["padding"], case["dilation"],
                           case["output_padding"], case["groups"])
        exp = np.array(case["y"], dtype=np.float64).reshape(case["y_shape"])
        assert y.shape == exp.shape, (f, y.shape, exp.shape)
        assert np.array_equal(y, exp), (f, y.ravel(), exp.ravel())
        n += 1
    assert n >= 7


def check_output_shapes(orc):
    case = json.load(open(os.path.join(GOLDEN_DIR, "example_shapes.json")))
    for c in case["cases"]:
        got = orc.out_shape(c["x_shape"], c["w_shape"], c["stride"], c["padding"],
                            c["dilation"], c["output_padding"], c["groups"])
        assert list(got) == c["y_shape"], (c, got)
    # and the full pass returns that shape (small cases only)
    c = case["cases"][0]
    y, _ = orc.forward(np.ones(c["x_shape"]), np.ones(c["w_shape"]))
    assert list(y.shape) == c["y_shape"]


def check_asymmetric_sizes(orc):
    """Sizes with a low and a high padding per axis (the AWS Neuron
    conv3d_transpose page's padding parameter), worked by hand from
    O = (I-1)*s - (p_lo + p_hi) + d*(k-1) + op + 1."""
    cases = [
        # (x_shape, w_shape, stride, padding pairs, dilation, output_padding, groups, y_shape)
        ((1, 1, 5), (1, 1, 3), (2,), ((1, 0),), (1,), (0,), 1, (1, 1, 10)),
        ((1, 1, 5), (1, 1, 3), (2,), ((0, 1),), (1,), (0,), 1, (1, 1, 10)),
        ((1, 2, 4, 6), (2, 3, 3, 2), (2, 3), ((0, 2), (1, 0)), (1, 2), (1, 0), 1, (1, 3, 8, 17)),
        ((2, 4, 3, 3, 3), (4, 1, 2, 2, 2), (1, 2, 2), ((0, 1), (1, 1), (2, 0)), (1, 1, 1),
         (0, 1, 0), 4, (2, 4, 3, 5, 4)),
    ]
    for xs, ws, st, pad, dl, op, g, ys in cases:
        assert tuple(orc.out_shape(xs, ws, st, pad, dl, op, g)) == ys, (xs, ws, pad)
    # equal ends give the symmetric size
    assert orc.out_shape((1, 1, 5), (1, 1, 3), 2, ((1, 1),), 1, 0) == \
        orc.out_shape((1, 1, 5), (1, 1, 3), 2, 1, 1, 0)


def check_asymmetric_window(orc):
    """Low padding p_lo drops the first p_lo outputs and high padding p_hi the
    last p_hi of the unpadded result, so the padded output is the window
    [p_lo, p_lo + O) of the p = 0 output, bit for bit."""
    rng = np.random.default_rng(22)
    for prm in random_grid(rng, 40):
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ph=prm["ph"])
        y, sc = orc.forward(x, w, b, **kw)
        kw0 = dict(kw, padding=0)
        y0, sc0 = orc.forward(x, w, b, **kw0)
        win = (slice(None), slice(None)) + tuple(
            slice(prm["p"][a], prm["p"][a] + y.shape[2 + a]) for a in range(prm["nd"]))
        assert all(y0.shape[2 + a] - y.shape[2 + a] == prm["p"][a] + prm["ph"][a]
                   for a in range(prm["nd"]))
        assert np.array_equal(y, y0[win]) and np.array_equal(sc, sc0[win])


def check_full_scatter_is_full_convolution(orc):
    rng = np.random.default_rng(11)
    for shape_x, shape_w in [((7,), (3,)), ((1,), (4,)), ((5, 4), (3, 2)), ((3, 4, 2), (2, 3, 2))]:
        x = rng.standard_normal(shape_x)
        w = rng.standard_normal(shape_w)
        y, _ = orc.forward(x[None, None], w[None, None])
        ref = scipy.signal.convolve(x, w, mode="full", method="direct")
        _close(y[0, 0], ref)


def check_stamp_is_kron(orc):
    rng = np.random.default_rng(12)
    for shape_x, shape_w in [((5,), (3,)), ((3, 4), (2, 3)), ((2, 3, 2), (2, 2, 3))]:
        x = rng.standard_normal(shape_x)
        w = rng.standard_normal(shape_w)
        y, _ = orc.forward(x[None, None], w[None, None], stride=shape_w)
        _close(y[0, 0], np.kron(x, w))


def check_pointwise_is_matmul(orc):
    rng = np.random.default_rng(13)
    for groups in (1, 2):
        B, Cig, Cog, H, W = 2, 3, 4, 5, 6
        x = rng.standard_normal((B, Cig * groups, H, W))
        w = rng.standard_normal((Cig * groups, Cog, 1, 1))
        b = rng.standard_normal(Cog * groups)
        y, _ = orc.forward(x, w, b, groups=groups)
        ref = np.empty((B, Cog * groups, H, W))
        for g in range(groups):
            wg = w[g * Cig:(g + 1) * Cig, :, 0, 0]  # [Cig, Cog]
            xg = x[:, g * Cig:(g + 1) * Cig].reshape(B, Cig, H * W)
            ref[:, g * Cog:(g + 1) * Cog] = np.matmul(wg.T, xg).reshape(B, Cog, H, W)
        ref += b[None, :, None, None]
        _close(y, ref)
    # kernel 1 with stride 3 and output_padding 2: zero-inserted upsample, the
    # two trailing positions hold the bias only
    x = rng.standard_normal((1, 2, 4))
    w = rng.standard_normal((2, 3, 1))
    b = rng.standard_normal(3)
    y, _ = orc.forward(x, w, b, stride=3, output_padding=2)
    assert y.shape == (1, 3, 12)
    ref = np.repeat(b[None, :, None], 12, axis=2).astype(np.float64)
    ref[0, :, 0:12:3] += np.matmul(w[:, :, 0].T, x[0])
    _close(y, ref)


def check_lowering_equivalence(orc):
    rng = np.random.default_rng(14)
    for prm in random_grid(rng, 60):
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ph=prm["ph"])
        y, _ = orc.forward(x, w, b, **kw)
        ref = lowered_reference(x, w, b, prm["s"], prm["p"], prm["d"], prm["op"], prm["groups"],
                                prm["ph"])
        _close(y, ref)


def check_adjoint_identity(orc):
    rng = np.random.default_rng(15)
    for prm in random_grid(rng, 40):
        x, w, _, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], bias=False, ph=prm["ph"])
        y, _ = orc.forward(x, w, None, **kw)
        yr = rng.standard_normal(y.shape)
        lhs = float(np.sum(y * yr))
        back = forward_conv_gather(yr, w, prm["s"], prm["p"], prm["d"], prm["I"], prm["groups"])
        rhs = float(np.sum(x * back))
        mag = float(np.sum(np.abs(x) * forward_conv_gather(np.abs(yr), np.abs(w), prm["s"],
                                                            prm["p"], prm["d"], prm["I"],
                                                            prm["groups"])))
        assert abs(lhs - rhs) <= 1e-12 * (mag + 1.0), (prm, lhs, rhs)


def check_groups_concatenate(orc):
    rng = np.random.default_rng(16)
    for prm in random_grid(rng, 20):
        if prm["groups"] == 1:
            continue
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ph=prm["ph"])
        y, _ = orc.forward(x, w, b, **kw)
        G, Cig, Cog = prm["groups"], prm["Ci"] // prm["groups"], prm["Cog"]
        parts = []
        for g in range(G):
            kw1 = dict(kw, groups=1)
            yg, _ = orc.forward(x[:, g * Cig:(g + 1) * Cig], w[g * Cig:(g + 1) * Cig],
                                b[g * Cog:(g + 1) * Cog], **kw1)
            parts.append(yg)
        assert np.array_equal(y, np.concatenate(parts, axis=1))


def check_bias_linearity_and_mass(orc):
    rng = np.random.default_rng(17)
    for prm in random_grid(rng, 30):
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ints=True, ph=prm["ph"])
        nd = prm["nd"]
        y_b, _ = orc.forward(x, w, b, **kw)
        y_0, _ = orc.forward(x, w, None, **kw)
        assert np.array_equal(y_b - y_0, np.broadcast_to(b.reshape((1, -1) + (1,) * nd), y_0.shape))
        x2 = rng.integers(-4, 5, size=x.shape).astype(np.float64)
        w2 = rng.integers(-4, 5, size=w.shape).astype(np.float64)
        assert np.array_equal(orc.forward(x + x2, w, None, **kw)[0], y_0 + orc.forward(x2, w, None, **kw)[0])
        assert np.array_equal(orc.forward(x, w + w2, None, **kw)[0], y_0 + orc.forward(x, w2, None, **kw)[0])
        # with padding 0 nothing is cropped: every product lands in the output
        kw0 = dict(kw, padding=(0,) * nd)
        y, _ = orc.forward(x, w, None, **kw0)
        G, Cig, Cog = prm["groups"], prm["Ci"] // prm["groups"], prm["Cog"]
        xs = x.reshape(x.shape[0], x.shape[1], -1).sum(axis=2)  # [B, Ci]
        ws = w.reshape(w.shape[0], w.shape[1], -1).sum(axis=2)  # [Ci, Cog]
        for g in range(G):
            tot = y[:, g * Cog:(g + 1) * Cog].reshape(y.shape[0], Cog, -1).sum(axis=2)
            ref = xs[:, g * Cig:(g + 1) * Cig] @ ws[g * Cig:(g + 1) * Cig]
            assert np.array_equal(tot, ref), (prm, tot, ref)


def check_brute_force(orc):
    rng = np.random.default_rng(18)
    for prm in random_grid(rng, 25, nds=(1, 2)):
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ph=prm["ph"])
        y, _ = orc.forward(x, w, b, **kw)
        ref = brute_force(x, w, b, prm["s"], prm["p"], prm["d"], prm["op"], prm["groups"],
                          prm["ph"])
        _close(y, ref)


def check_scale_is_abs_convt(orc):
    rng = np.random.default_rng(19)
    for prm in random_grid(rng, 20):
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ph=prm["ph"])
        _, sc = orc.forward(x, w, b, **kw)
        ref, _ = orc.forward(np.abs(x), np.abs(w), None, **kw)
        _close(sc, ref)
        ref2 = lowered_reference(np.abs(x), np.abs(w), None, prm["s"], prm["p"], prm["d"],
                                 prm["op"], prm["groups"], prm["ph"])
        _close(sc, ref2)


def check_points_match_forward(orc):
    rng = np.random.default_rng(20)
    for prm in random_grid(rng, 30):
        x, w, b, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ph=prm["ph"])
        y, sc = orc.forward(x, w, b, **kw)
        pts = np.array(list(itertools.product(*[range(t) for t in y.shape])), dtype=np.int64)
        yv, sv = orc.points(x, w, b, pts, **kw)
        _close(yv, y.ravel())
        _close(sv, sc.ravel())


def check_thread_count_independent(orc):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 6, 9, 7))
    w = rng.standard_normal((6, 5, 3, 4))
    b = rng.standard_normal(10)
    kw = dict(stride=(2, 3), padding=(1, 2), dilation=(1, 2), output_padding=(1, 0), groups=2)
    y1, s1 = orc.forward(x, w, b, nthreads=1, **kw)
    y8, s8 = orc.forward(x, w, b, nthreads=8, **kw)
    assert np.array_equal(y1, y8) and np.array_equal(s1, s8)


def check_rejects_ill_formed(orc):
    bad = [
        dict(x=(1, 1, 1), w=(1, 1, 1), s=(1,), p=(1,), d=(1,), op=(0,), g=1),   # O = -1
        dict(x=(1, 3, 4), w=(3, 1, 2), s=(1,), p=(0,), d=(1,), op=(0,), g=2),   # 2 does not divide 3
        dict(x=(1, 2, 4), w=(3, 1, 2), s=(1,), p=(0,), d=(1,), op=(0,), g=1),   # C_in mismatch
        dict(x=(1, 2, 4), w=(2, 1, 2), s=(0,), p=(0,), d=(1,), op=(0,), g=1),   # stride 0
        dict(x=(1, 1, 4), w=(1, 1, 2), s=(1,), p=((0, -1),), d=(1,), op=(0,), g=1),  # p_hi < 0
        dict(x=(1, 1, 2), w=(1, 1, 2), s=(1,), p=((0, 3),), d=(1,), op=(0,), g=1),   # O = 0
    ]
    for c in bad:
        try:
            orc.out_shape(c["x"], c["w"], c["s"], c["p"], c["d"], c["op"], c["g"])
        except ValueError:
            continue
        raise AssertionError(f"accepted {c}")


# ---------------------------------------------------------------------------
# Backward data (input gradient)
# ---------------------------------------------------------------------------

def check_bwd_is_jacobian_transpose(orc):
    """y is linear in x: column j of its Jacobian is the forward pass of the
    unit input e_j (no bias). The input gradient must be J^T dy, exactly on
    integer data."""
    rng = np.random.default_rng(30)
    for prm in random_grid(rng, 14):
        x, w, _, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], ints=True, bias=False, ph=prm["ph"])
        y0, _ = orc.forward(x, w, None, with_scale=False, **kw)
        cols = []
        for j in range(x.size):
            e = np.zeros(x.size)
            e[j] = 1.0
            cols.append(orc.forward(e.reshape(x.shape), w, None, with_scale=False, **kw)[0].ravel())
        J = np.stack(cols, axis=1)  # [y.size, x.size]
        dy = rng.integers(-4, 5, size=y0.shape).astype(np.float64)
        dx, _ = orc.backward_data(dy, w, x.shape, **kw)
        assert np.array_equal(dx.ravel(), J.T @ dy.ravel()), prm


def check_bwd_adjoint_identity(orc):
    """<convT(x, W), dy> = <x, dx(dy, W)> on random real data."""
    rng = np.random.default_rng(31)
    for prm in random_grid(rng, 40):
        x, w, _, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], bias=False, ph=prm["ph"])
        y, _ = orc.forward(x, w, None, with_scale=False, **kw)
        dy = rng.standard_normal(y.shape)
        dx, sc = orc.backward_data(dy, w, x.shape, **kw)
        lhs, rhs = float(np.sum(y * dy)), float(np.sum(x * dx))
        mag = float(np.sum(np.abs(x) * sc)) + 1.0
        assert abs(lhs - rhs) <= 1e-12 * mag, (prm, lhs, rhs)


def check_bwd_valid_correlation(orc):
    """Stride 1, no padding, dilation 1: the forward pass is a full
    convolution, so its input gradient is the valid cross-correlation of dy
    with the kernel (scipy)."""
    rng = np.random.default_rng(32)
    for shape_x, shape_w in [((7,), (3,)), ((5, 4), (3, 2)), ((3, 4, 2), (2, 3, 2))]:
        w = rng.standard_normal(shape_w)
        oshape = tuple(a + b - 1 for a, b in zip(shape_x, shape_w))
        dy = rng.standard_normal(oshape)
        dx, _ = orc.backward_data(dy[None, None], w[None, None], (1, 1) + shape_x)
        ref = scipy.signal.correlate(dy, w, mode="valid", method="direct")
        _close(dx[0, 0], ref)


def brute_force_bwd(dy, w, x_shape, s, p, d, groups):
    """dx by enumerating every (input position, tap, output channel) in
    Python: dx[b, ci, i] collects dy[b, oc, o] * W[ci, oc - g*Cog, kk] for
    o = i*s - p + kk*d inside dy."""
    nd = len(x_shape) - 2
    B, Ci = x_shape[:2]
    Cig, Cog = Ci // groups, w.shape[1]
    k = w.shape[2:]
    I = x_shape[2:]
    O = dy.shape[2:]
    dx = np.zeros(x_shape)
    for b in range(B):
        for ci in range(Ci):
            g = ci // Cig
            for i in itertools.product(*[range(t) for t in I]):
                acc = 0.0
                for oc in range(g * Cog, (g + 1) * Cog):
                    for kk in itertools.product(*[range(t) for t in k]):
                        o = tuple(i[a] * s[a] - p[a] + kk[a] * d[a] for a in range(nd))
                        if all(0 <= o[a] < O[a] for a in range(nd)):
                            acc += float(dy[(b, oc) + o]) * float(w[(ci, oc - g * Cog) + kk])
                dx[(b, ci) + i] = acc
    return dx


def check_bwd_brute_force(orc):
    rng = np.random.default_rng(33)
    for prm in random_grid(rng, 20, nds=(1, 2)):
        x, w, _, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], bias=False, ph=prm["ph"])
        oshape = orc.out_shape(x.shape, w.shape, kw["stride"], kw["padding"], kw["dilation"],
                               kw["output_padding"], kw["groups"])
        dy = rng.standard_normal(oshape)
        dx, _ = orc.backward_data(dy, w, x.shape, **kw)
        _close(dx, brute_force_bwd(dy, w, x.shape, prm["s"], prm["p"], prm["d"], prm["groups"]))


def check_bwd_points_and_scale(orc):
    """The point form equals the full pass, and the magnitude sum equals the
    input gradient of |dy| with |W|."""
    rng = np.random.default_rng(34)
    for prm in random_grid(rng, 25):
        x, w, _, kw = _rand_problem(rng, prm["nd"], prm["B"], prm["Ci"], prm["Cog"],
                                    prm["groups"], prm["I"], prm["k"], prm["s"], prm["p"],
                                    prm["d"], prm["op"], bias=False, ph=prm["ph"])
        oshape = orc.out_shape(x.shape, w.shape, kw["stride"], kw["padding"], kw["dilation"],
                               kw["output_padding"], kw["groups"])
        dy = rng.standard_normal(oshape)
        dx, sc = orc.backward_data(dy, w, x.shape, **kw)
        pts = np.array(list(itertools.product(*[range(t) for t in x.shape])), dtype=np.int64)
        xv, sv = orc.backward_data_points(dy, w, x.shape, pts, **kw)
        _close(xv, dx.ravel())
        _close(sv, sc.ravel())
        ref, _ = orc.backward_data(np.abs(dy), np.abs(w), x.shape, **kw)
        _close(sc, ref)


# ---------------------------------------------------------------------------
# Activation (applied after the bias)
# ---------------------------------------------------------------------------

def check_activation_closed_forms(orc):
    """Each activation against its textbook form through numpy / scipy, over
    values from deep negative to deep positive, and its exact special values."""
    from scipy.special import erf, expit
    v = np.concatenate([np.linspace(-40.0, 40.0, 4001), [-745.0, -1e-300, 0.0, 1e-300, 709.0]])
    ref = {
        1: np.maximum(v, 0.0),
        2: expit(v),
        3: np.tanh(v),
        4: v * expit(v),
        5: 0.5 * v * (1.0 + erf(v / np.sqrt(2.0))),
    }
    assert np.array_equal(orc.activation(0, v), v)
    for a, r in ref.items():
        got = orc.activation(a, v)
        assert np.all(np.abs(got - r) <= 1e-13 * (np.abs(r) + 1e-300) + 1e-300), a
    z = np.zeros(1)
    assert orc.activation(2, z)[0] == 0.5 and orc.activation(3, z)[0] == 0.0
    assert orc.activation(4, z)[0] == 0.0 and orc.activation(5, z)[0] == 0.0
    try:
        orc.activation(6, z)
    except ValueError:
        pass
    else:
        raise AssertionError("activation code 6 accepted")


def check_activation_follows_bias(orc):
    """The activation applies to each output after the bias is added: a
    bias shift moves the pre-activation value, which only ReLU's flat side
    can hide."""
    from scipy.special import expit
    rng = np.random.default_rng(40)
    x = rng.standard_normal((2, 4, 5, 6))
    w = rng.standard_normal((4, 3, 3, 3))
    b = rng.standard_normal(3) * 3.0
    kw = dict(stride=2, padding=1, dilation=1, output_padding=1, groups=1)
    y0, _ = orc.forward(x, w, b, **kw)
    y2, _ = orc.forward(x, w, b, activation=2, **kw)
    _close(y2, expit(y0))
    p, _ = orc.points(x, w, b, np.array([[1, 2, 3, 4], [0, 0, 0, 0]]), activation=2, **kw)
    _close(p, expit(y0[(np.array([1, 0]), np.array([2, 0]), np.array([3, 0]), np.array([4, 0]))]))


ALL_CHECKS = [
    check_golden_cases,
    check_output_shapes,
    check_asymmetric_sizes,
    check_asymmetric_window,
    check_full_scatter_is_full_convolution,
    check_stamp_is_kron,
    check_pointwise_is_matmul,
    check_lowering_equivalence,
    check_adjoint_identity,
    check_groups_concatenate,
    check_bias_linearity_and_mass,
    check_brute_force,
    check_scale_is_abs_convt,
    check_points_match_forward,
    check_thread_count_independent,
    check_rejects_ill_formed,
    check_bwd_is_jacobian_transpose,
    check_bwd_adjoint_identity,
    check_bwd_valid_correlation,
    check_bwd_brute_force,
    check_bwd_points_and_scale,
    check_activation_closed_forms,
    check_activation_follows_bias,
]
