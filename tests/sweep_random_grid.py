# Robustness sweep (run by hand on a GPU, not collected by pytest): larger
# random grids than the committed tests, from new seeds, through the GPU
# test helpers: forward (symmetric and asymmetric pads) and backward, with a
# third of the cases in float16, every route that serves each; prints
# failures with their parameters.
#     python tests/sweep_random_grid.py <cases per kind> <seed>
import os, sys, traceback
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import numpy as np
import convt_forward_amd as C
from tests import test_gpu_parity as P, test_gpu_backward as Bk

n, seed0 = int(sys.argv[1]), int(sys.argv[2])
fails = []

def f16ify(cases):
    for i, prm in enumerate(cases):
        if i % 3 == 2:
            prm["dtype"] = "f16"
    return cases

def bwd_case(prm, tag):
    xs = (prm["B"], prm["Ci"]) + tuple(prm["I"])
    ws = (prm["Ci"], prm["Cog"]) + tuple(prm["k"])
    pad = tuple(prm["p"]) if prm["p"] == prm["ph"] else tuple(zip(prm["p"], prm["ph"]))
    p = dict(stride=tuple(prm["s"]), padding=pad, dilation=tuple(prm["d"]),
             output_padding=tuple(prm["op"]), groups=prm["groups"])
    for route in Bk.ROUTES:
        try:
            C.get_plan(xs, ws, p["stride"], p["padding"], p["dilation"], p["output_padding"],
                       p["groups"], False, prm["dtype"], "auto", route)
        except C.ConvtError as e:
            assert e.status == 2
            continue
        Bk.check_bwd_full(xs, ws, p, prm["dtype"], route, prm["seed"], tag)

sets = [("fwd", f16ify(P.grid_cases(n, seed0))),
        ("fwd_asym", f16ify(P.grid_cases(n, seed0 + 1, asym=True))),
        ("bwd", f16ify(Bk.grid_cases(n, seed0 + 2)))]
for kind, cases in sets:
    for i, prm in enumerate(cases):
        tag = f"{kind}[{i}]"
        try:
            if kind == "bwd":
                bwd_case(prm, tag)
            else:
                P.run_grid_case(prm, tag)
        except Exception as e:
            fails.append((tag, prm, repr(e)[:300]))
            print("FAIL", tag, prm, repr(e)[:300], flush=True)
        if i % 25 == 24:
            print(f"{kind}: {i + 1}/{len(cases)} done, failures so far {len(fails)}", flush=True)
print(f"sweep done: {sum(len(c) for _, c in sets)} cases, {len(fails)} failures", flush=True)
