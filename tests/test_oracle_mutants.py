"""CPU tests: planted mistakes in the oracle's C source must fail a pin.

Each mutant below is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a wrong group or size formula). It is compiled from a
modified copy of oracle/convt_oracle.c and the whole pin suite runs against it
in a child process; the mutant counts as caught when that process fails. Every
mutation keeps all memory accesses in bounds.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "convt_oracle.c")

# The forward scatter's inner loops; mutants of lines that also occur in the
# backward-data loops are applied inside this block only.
FWD = ("++i2) {\n                const double xv = xp[(i0 * pb.I[1] + i1) * pb.I[2] + i2];",
       "const double wv = wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];")

MUTANTS = [
    ("bias dropped", "const double b0 = bias ? bias[oc] : 0.0;", "const double b0 = 0.0;"),
    ("padding sign", "const int64_t o2 = i2 * pb.S[2] - pb.P[2] + k2 * pb.D[2];",
     "const int64_t o2 = i2 * pb.S[2] + pb.P[2] + k2 * pb.D[2];", FWD),
    ("dilation dropped", "const int64_t o1 = i1 * pb.S[1] - pb.P[1] + k1 * pb.D[1];",
     "const int64_t o1 = i1 * pb.S[1] - pb.P[1] + k1;", FWD),
    ("stride of wrong axis", "const int64_t o2 = i2 * pb.S[2] - pb.P[2] + k2 * pb.D[2];",
     "const int64_t o2 = i2 * pb.S[1] - pb.P[2] + k2 * pb.D[2];", FWD),
    ("taps flipped", "const double wv = wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];\n"
     "                            const int64_t o =",
     "const double wv = wp[(k0 * pb.K[1] + k1) * pb.K[2] + (pb.K[2] - 1 - k2)];\n"
     "                            const int64_t o ="),
    ("input channel reversed", "const double *xp = x + (b * pb.Ci + ci) * isz;\n            const double *wp = w + (ci * pb.Cog + ocl) * ksz;\n            for (int64_t i0",
     "const double *xp = x + (b * pb.Ci + (pb.Ci - 1 - ci)) * isz;\n            const double *wp = w + (ci * pb.Cog + ocl) * ksz;\n            for (int64_t i0"),
    ("wrong group of an output channel", "const int64_t g = oc / pb.Cog;", "const int64_t g = oc % pb.G;"),
    ("output_padding ignored in size", "return (in - 1) * s - (p + ph) + d * (k - 1) + op + 1;",
     "return (in - 1) * s - (p + ph) + d * (k - 1) + 1;"),
    ("padding counted once in size", "return (in - 1) * s - (p + ph) + d * (k - 1) + op + 1;",
     "return (in - 1) * s - p + d * (k - 1) + op + 1;"),
    ("low padding counted twice in size", "return (in - 1) * s - (p + ph) + d * (k - 1) + op + 1;",
     "return (in - 1) * s - 2 * p + d * (k - 1) + op + 1;"),
    ("high padding read as the low one", "pb->PH[a] = padding_end ? padding_end[j] : padding[j];",
     "pb->PH[a] = padding[j];"),
    ("high padding shifts the outputs", "const int64_t o2 = i2 * pb.S[2] - pb.P[2] + k2 * pb.D[2];",
     "const int64_t o2 = i2 * pb.S[2] - pb.PH[2] + k2 * pb.D[2];", FWD),
    ("high padding shifts the point form", "const int64_t t1 = o[1] + pb.P[1] - k1 * pb.D[1];",
     "const int64_t t1 = o[1] + pb.PH[1] - k1 * pb.D[1];"),
    ("first output position dropped", "if (o2 < 0 || o2 >= pb.O[2]) continue;",
     "if (o2 < 1 || o2 >= pb.O[2]) continue;", FWD),
    ("signed magnitude", "if (sp) sp[o] += fabs(xv * wv);", "if (sp) sp[o] += xv * wv;"),
    ("negative remainder in the point form", "if (t2 % pb.S[2] != 0) continue;",
     "if (t2 % pb.S[2] > 0) continue;"),
    ("weight channel offset transposed",
     "const double *wp = w + (ci * pb.Cog + ocl) * ksz;\n            for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {\n"
     "                const int64_t t0",
     "const double *wp = w + ((ci - g * pb.Cig) * pb.Cog + ocl) * ksz;\n            for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {\n"
     "                const int64_t t0"),
    # backward data (input gradient)
    ("bwd: wrong group of an input channel", "const int64_t g = ci / pb.Cig;",
     "const int64_t g = ci % pb.G;"),
    ("bwd: taps flipped",
     "const double t = yp[(o0 * pb.O[1] + o1) * pb.O[2] + o2] *\n"
     "                                             wp[(k0 * pb.K[1] + k1) * pb.K[2] + k2];",
     "const double t = yp[(o0 * pb.O[1] + o1) * pb.O[2] + o2] *\n"
     "                                             wp[(k0 * pb.K[1] + k1) * pb.K[2] + (pb.K[2] - 1 - k2)];"),
    ("bwd: dy channel outside the group",
     "const double *yp = dy + (b * pb.Co + g * pb.Cog + ocl) * osz;\n                const double *wp",
     "const double *yp = dy + (b * pb.Co + ocl) * osz;\n                const double *wp"),
    ("bwd: padding sign",
     "ksz;\n                for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {\n"
     "                    const int64_t o0 = i0 * pb.S[0] - pb.P[0] + k0 * pb.D[0];",
     "ksz;\n                for (int64_t k0 = 0; k0 < pb.K[0]; ++k0) {\n"
     "                    const int64_t o0 = i0 * pb.S[0] + pb.P[0] + k0 * pb.D[0];"),
    ("bwd points: dropped dilation", "const int64_t o0 = i[0] * pb.S[0] - pb.P[0] + k0 * pb.D[0];",
     "const int64_t o0 = i[0] * pb.S[0] - pb.P[0] + k0;"),
    ("bwd points: signed magnitude", "acc += t;\n                        mag += fabs(t);",
     "acc += t;\n                        mag += t;"),
    # activation
    ("sigmoid sign", "case 2: r = 1.0 / (1.0 + exp(-v)); break;",
     "case 2: r = 1.0 / (1.0 + exp(v)); break;"),
    ("GELU by its tanh approximation", "case 5: r = 0.5 * v * (1.0 + erf(v / sqrt(2.0))); break;",
     "case 5: r = 0.5 * v * (1.0 + tanh(0.7978845608028654 * (v + 0.044715 * v * v * v))); break;"),
    ("leaky ReLU", "case 1: r = v > 0.0 ? v : 0.0; break;", "case 1: r = v > 0.0 ? v : 0.01 * v; break;"),
    ("SiLU with the sigmoid of -v", "case 4: r = v / (1.0 + exp(-v)); break;",
     "case 4: r = v / (1.0 + exp(v)); break;"),
    ("tanh dropped", "case 3: r = tanh(v); break;", "case 3: r = v; break;"),
    ("bwd: high padding shifts the gradient",
     "                            const int64_t o2 = i2 * pb.S[2] - pb.P[2] + k2 * pb.D[2];\n"
     "                            if (o2 < 0 || o2 >= pb.O[2]) continue;\n"
     "                            const double t",
     "                            const int64_t o2 = i2 * pb.S[2] - pb.PH[2] + k2 * pb.D[2];\n"
     "                            if (o2 < 0 || o2 >= pb.O[2]) continue;\n"
     "                            const double t"),
]


def mutate(src, name, old, new, scope=None):
    """src with `old` replaced by `new`; `old` must occur exactly once in the
    source, or, with a scope (first, last), exactly once in the unique block
    from first to last."""
    if scope is None:
        assert src.count(old) == 1, f"mutation anchor for {name!r} not found exactly once"
        return src.replace(old, new)
    first, last = scope
    assert src.count(first) == 1, f"scope start for {name!r} not unique"
    a = src.index(first)
    b = src.index(last, a) + len(last)
    block = src[a:b]
    assert block.count(old) == 1, f"mutation anchor for {name!r} not found once in its scope"
    return src[:a] + block.replace(old, new) + src[b:]


@pytest.mark.parametrize("m", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, m):
    name = m[0]
    src = open(SRC).read()
    msrc = tmp_path / "mutant.c"
    msrc.write_text(mutate(src, *m))
    lib = oracle.build(force=True, src=str(msrc), out=str(tmp_path / "libmutant.so"))
    code = ("import sys; sys.path.insert(0, %r); import oracle; from tests import oracle_pins; "
            "o = oracle.Oracle(%r); [c(o) for c in oracle_pins.ALL_CHECKS]" % (ROOT, lib))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name!r} passed every pin"
